/*
 * attn.h - C ABI of the exact tiled attention library for AMD Instinct MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention over packed ragged sequences
 * as an I/O-aware tiled HIP kernel: logits Q K^T, exclusion of disallowed pairs, an
 * online-softmax rescale, P V, and a saved log-sum-exp; the backward pass recomputes P
 * from that log-sum-exp and produces dQ, dK, dV.
 *
 * Operator (per query token t of sequence s, query head h, K/V head g = h / (Hq / Hkv)):
 *     O[t,h,:]  = sum_u p(t,u) V[u,g,:],   p(t,u) = exp(scale q.k_u - LSE[h,t]) if allowed
 *     LSE[h,t]  = log sum_{allowed u} exp(scale q_t.k_u)       (natural log)
 * A row with no allowed key gives O = +0.0 and LSE = -inf.
 *   - Efficient Attention: Formal Correctness, "The FlashAttention Proof": the tiled kernel
 *     computes exactly the naive specification; the online recurrence keeps a running max,
 *     rescales the denominator and accumulator when it moves, and divides at the end.
 *   - Causal Mask and Ragged Sequence Layouts, sections 1-4: a pair is allowed only inside
 *     one sequence, compared on in-sequence positions (never on packed offsets); out-of-
 *     range tile lanes never enter the max, denominator or gradient reductions; causal
 *     alignment is an explicit choice (top-left: j <= i; bottom-right: j <= i + Nk - Nq);
 *     all-masked rows output zero.
 *   - Attention Algorithm Error and Complexity Tests, section 3: GQA query heads share K/V
 *     heads by consecutive grouping and their K/V gradients are summed.
 *   - Window (a bounded window is named in the same page's fifth section without a
 *     formula): width W > 0 keeps keys with position in (end - W, end], where end is the
 *     aligned diagonal (pos_q for top-left, pos_q + Nk - Nq for bottom-right).
 *
 * Layout (all row-major, contiguous, head_dim fastest):
 *   q, out, dout, dq : [total_q, Hq, head_dim]     element type `dtype`
 *   k, v, dk, dv     : [total_k, Hkv, head_dim]    element type `dtype`
 *   lse              : [Hq, total_q]               float32, natural-log units
 *   cu_seqlens_q/k   : [num_seqs + 1] int32, cu[0] = 0, nondecreasing, cu[num_seqs] =
 *                      total_q / total_k. Sequence s owns tokens [cu[s], cu[s+1]); zero-
 *                      length sequences are allowed.
 *
 * Ownership: every pointer is caller-owned DEVICE memory (cu_seqlens included). The
 * library never allocates or frees memory and keeps no pointer after a call returns. Calls
 * are asynchronous on `stream` (a hipStream_t; NULL = the default stream): results are
 * valid once that stream has been synchronised. Outputs must not alias inputs. Calls on
 * different streams are independent when their workspaces and outputs differ.
 *
 * Errors: every entry point validates its arguments on the host before launching anything
 * and returns ATTN_OK (0) or a negative attn_status; on error no output is written. There
 * is no fallback path: an unsupported combination is an error. Malformed cu_seqlens
 * contents (device memory, not read by the host) are undefined behaviour; attn_check_seqlens
 * detects them.
 */
#ifndef EXACT_ATTENTION_TILED_ATTN_H
#define EXACT_ATTENTION_TILED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_VERSION 110   /* 1.1.0 */

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL_PTR = -1,             /* a required pointer is NULL */
  ATTN_ERR_BAD_SHAPE = -2,            /* negative size, head_dim not 64/128, max_seqlen < 0 */
  ATTN_ERR_BAD_HEADS = -3,            /* Hq or Hkv < 1, or Hq % Hkv != 0 */
  ATTN_ERR_BAD_DTYPE = -4,            /* dtype not ATTN_BF16 / ATTN_F32 */
  ATTN_ERR_BAD_MASK = -5,             /* unknown mask_mode, or window > 0 without causal */
  ATTN_ERR_WORKSPACE_TOO_SMALL = -6,  /* workspace_bytes below the size query's answer */
  ATTN_ERR_UNSUPPORTED_DEVICE = -7,   /* current device is not gfx950 */
  ATTN_ERR_LAUNCH_FAILED = -8,        /* the HIP runtime rejected a kernel launch */
  ATTN_ERR_BAD_SCALE = -9,            /* scale is not finite */
  ATTN_ERR_BAD_PLAN = -10,            /* forced path / split count not usable for the shape */
  ATTN_ERR_BAD_RANGE = -11,           /* probe window outside the token ranges */
  ATTN_ERR_BAD_DROPOUT = -12,         /* dropout probability not in [0, 255.5/256) */
  ATTN_ERR_SCRATCH_TOO_SMALL = -13    /* attn_fwd_no_workspace: needs more than the scratch */
} attn_status;

enum attn_dtype { ATTN_BF16 = 0, ATTN_F32 = 1 };

enum attn_mask_mode {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_CAUSAL_TOP_LEFT = 1,      /* key j allowed iff j <= i */
  ATTN_MASK_CAUSAL_BOTTOM_RIGHT = 2   /* key j allowed iff j <= i + Nk - Nq */
};

/* Forward paths. AUTO picks PREFILL or SPLITK from the shape; the choice is reported by
 * attn_describe_plan. */
enum attn_path { ATTN_PATH_AUTO = 0, ATTN_PATH_PREFILL = 1, ATTN_PATH_SPLITK = 2 };

/*
 * attn_fwd - forward pass: writes out [total_q, Hq, d] and lse [Hq, total_q].
 *   q, k, v          inputs (layout above), element type `dtype`
 *   num_seqs         number of packed sequences (0 = nothing to do, returns ATTN_OK)
 *   total_q/total_k  token counts (= cu[num_seqs])
 *   max_seqlen_q/k   host-side upper bounds of the per-sequence lengths (used for grid
 *                    sizing; a bound below the true maximum is undefined behaviour)
 *   num_heads_q/kv   Hq, Hkv with Hq % Hkv == 0
 *   head_dim         64 or 128
 *   scale            finite multiplier of q.k (usually 1/sqrt(head_dim))
 *   mask_mode        attn_mask_mode; window > 0 needs a causal mode, window <= 0 = none
 *   workspace        device scratch of at least attn_fwd_workspace_size(...) bytes (may be
 *                    NULL when that size is 0); its contents need no initialisation. The
 *                    split-K plan keeps its partial results there and sizes its grid by the
 *                    CU count of the current device, so query the size with the device
 *                    current that will run the call. A prefill over sequences of unequal
 *                    lengths keeps its cost-sorted tile order there (4 bytes per query-tile
 *                    slot: total_q / 128 + num_seqs slots); one of equal lengths needs none.
 */
int attn_fwd(const void* q, const void* k, const void* v,
             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
             int32_t num_seqs, int32_t total_q, int32_t total_k,
             int32_t max_seqlen_q, int32_t max_seqlen_k,
             int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, int32_t dtype,
             float scale, int32_t mask_mode, int32_t window,
             void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

size_t attn_fwd_workspace_size(int32_t num_seqs, int32_t total_q, int32_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                               int32_t dtype, int32_t mask_mode, int32_t window);

/*
 * attn_fwd_no_workspace - attn_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Instead of a caller workspace it uses a fixed scratch array of
 * ATTN_SCRATCH_BYTES that the library holds in device memory, one per GPU, until the
 * process ends; it calls no allocator (no hipMalloc, hipFree or allocating library routine).
 * Same arguments, plan, kernels and results as attn_fwd with ATTN_PATH_AUTO.
 *   Limit: a call whose plan needs more than ATTN_SCRATCH_BYTES of workspace (what
 *          attn_fwd_workspace_size reports for it) returns ATTN_ERR_SCRATCH_TOO_SMALL before
 *          any launch; e.g. the split-K decode of 16 sequences x 32 query heads x 16 queries
 *          at head_dim 128 needs about 8.4 MiB.
 *   Concurrency: every call on one GPU shares that GPU's scratch, which keeps whatever the
 *          last call left there. Calls that overlap in time on one GPU (other streams, other
 *          threads) race on it; serialise them, or use attn_fwd with separate workspaces.
 */
#define ATTN_SCRATCH_BYTES (16u << 20)

int attn_fwd_no_workspace(const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int32_t num_seqs, int32_t total_q, int32_t total_k,
                          int32_t max_seqlen_q, int32_t max_seqlen_k,
                          int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                          int32_t dtype, float scale, int32_t mask_mode, int32_t window,
                          void* out, float* lse, void* stream);

/*
 * attn_fwd_ex / attn_fwd_ex_workspace_size - the forward pass with the path chosen by the
 * caller (ATTN_PATH_*) and, for SPLITK, the number of key-range blocks per (sequence,
 * K/V head) (0 = choose). Exists so tests and experiments can run both paths on the same
 * inputs; results of every path satisfy the same contract.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v,
                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                int32_t num_seqs, int32_t total_q, int32_t total_k,
                int32_t max_seqlen_q, int32_t max_seqlen_k,
                int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, int32_t dtype,
                float scale, int32_t mask_mode, int32_t window,
                int32_t path, int32_t num_splits,
                void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

size_t attn_fwd_ex_workspace_size(int32_t num_seqs, int32_t total_q, int32_t total_k,
                                  int32_t max_seqlen_q, int32_t max_seqlen_k,
                                  int32_t num_heads_q, int32_t num_heads_kv,
                                  int32_t head_dim, int32_t dtype, int32_t mask_mode,
                                  int32_t window, int32_t path, int32_t num_splits);

/*
 * attn_bwd - backward pass of attn_fwd for loss gradient dout: writes dq (like q) and
 * dk, dv (like k; summed over each GQA group). `out` and `lse` must be the forward's
 * outputs for the same inputs and the SAME mask arguments (the backward rebuilds the same
 * logical mask: Causal Mask and Ragged Sequence Layouts, section 6). Keys no query may
 * attend get dk = dv = 0; empty query rows get dq = 0.
 *   dtype            ATTN_BF16 or ATTN_F32 (the dtype of q, k, v, out, dout, dq, dk, dv);
 *                    fp32 products are exact with fp32 accumulation
 *   workspace        device scratch of at least attn_bwd_workspace_size(...) bytes
 *                    (8 * Hq * total_q rounded up to 256-byte pieces); no initialisation needed
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
             const void* dout, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
             int32_t num_seqs, int32_t total_q, int32_t total_k,
             int32_t max_seqlen_q, int32_t max_seqlen_k,
             int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, int32_t dtype,
             float scale, int32_t mask_mode, int32_t window,
             void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
             void* stream);

size_t attn_bwd_workspace_size(int32_t num_seqs, int32_t total_q, int32_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                               int32_t dtype, int32_t mask_mode, int32_t window);

/*
 * attn_fwd_dropout / attn_bwd_dropout - attn_fwd / attn_bwd with inverted dropout on the
 * attention weights. Dropout is a separate contract from the deterministic operator
 * (Attention Algorithm Error and Complexity Tests, section 1) whose realisation replays in
 * the backward and across packings by logical index (Causal Mask and Ragged Sequence
 * Layouts, section 6; same first page, section 4: gradients use the same realisation):
 *     O[t,h,:] = sum_u p(t,u) keep(s,h,i,j) / (1 - t8/256) V[u,g,:]
 * with p(t,u) and LSE exactly as for attn_fwd (the LSE is that of the undropped softmax).
 * keep(s,h,i,j) for sequence index s, query head h, in-sequence query position i and key
 * position j: byte j % 4 of output word i % 4 of Philox4x32-10 (Salmon et al., SC'11) at
 * counter (i / 4, j / 4, h, s) and key (seed & 0xffffffff, seed >> 32), kept iff that byte
 * is >= t8 = floor(256 * dropout_p + 0.5) (computed in double from the float argument).
 *   dropout_p   in [0, 255.5/256), else ATTN_ERR_BAD_DROPOUT; t8 = 0 without
 *               out_residual runs attn_fwd / attn_bwd unchanged
 *   seed        any 64-bit value; attn_bwd_dropout must get the forward's dropout_p and seed
 * The forward always runs the prefill path (bf16 or fp32) and needs the workspace of
 * attn_fwd_dropout_workspace_size; the backward (bf16 or fp32, like attn_bwd) needs
 * attn_bwd_workspace_size. Other arguments, ownership and errors as attn_fwd / attn_bwd.
 *   out_residual  optional (may be NULL), bf16 only (ATTN_ERR_BAD_DTYPE otherwise):
 *               [total_q, Hq, head_dim] bf16 like out. The forward writes x - bf16(x) for
 *               every output element x it rounds into out; given the same buffer, the
 *               backward forms D = rowsum(dO * O) from out + out_residual. Without it the
 *               bf16 backward with t8 > 0 computes D = sum_u P dP in a pass of its own (the
 *               stored output's rounding no longer cancels in dS once weights are dropped
 *               and rescaled), which costs a recomputation of S and dP; the residual trades
 *               that pass for one more output-sized tensor kept from the forward.
 *               With t8 = 0 and out_residual given, the pair is attn_fwd / attn_bwd (prefill
 *               path) with D formed from the unrounded output: the route for inputs where
 *               the stored output's rounding does not cancel in dS either (|scale| far above
 *               1/sqrt(head_dim), values with a large common offset), at the cost of an
 *               unpipelined forward with a second PV contraction. The backward must get the
 *               buffer its forward wrote: a residual never written gives wrong gradients.
 */
int attn_fwd_dropout(const void* q, const void* k, const void* v,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                     int32_t num_seqs, int32_t total_q, int32_t total_k,
                     int32_t max_seqlen_q, int32_t max_seqlen_k,
                     int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, int32_t dtype,
                     float scale, int32_t mask_mode, int32_t window,
                     float dropout_p, uint64_t seed,
                     void* out, float* lse, void* out_residual, void* workspace,
                     size_t workspace_bytes, void* stream);

size_t attn_fwd_dropout_workspace_size(int32_t num_seqs, int32_t total_q, int32_t total_k,
                                       int32_t max_seqlen_q, int32_t max_seqlen_k,
                                       int32_t num_heads_q, int32_t num_heads_kv,
                                       int32_t head_dim, int32_t dtype, int32_t mask_mode,
                                       int32_t window);

int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const void* out_residual, const void* dout,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                     int32_t num_seqs, int32_t total_q, int32_t total_k,
                     int32_t max_seqlen_q, int32_t max_seqlen_k,
                     int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, int32_t dtype,
                     float scale, int32_t mask_mode, int32_t window,
                     float dropout_p, uint64_t seed,
                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * attn_dropout_probe - runs the kernels' dropout realisation for sequence index seq and
 * query head head over in-sequence positions [q0, q0 + nq) x [k0, k0 + nk), in the lane
 * layout the kernels use: 64-lane waves on 32-aligned 32 x 32 blocks, once in the row form
 * of the forward and dQ kernels (a lane per query, key quads per register group) and once
 * in the column form of the dK/dV kernel (a lane per key). Writes keep[i * nk + j] (uint8,
 * device memory, nq * nk bytes): bit 0 = 1 if the row form keeps element (q0 + i, k0 + j),
 * bit 1 = the same for the column form; bits 2-7 are zero. Both bits agree for a correct
 * realisation: the flags are a function of logical indices only, so the backward regenerates
 * the forward's (Causal Mask and Ragged Sequence Layouts, sixth section). Exists so the
 * realisation can be tested bit-exactly. Positions are not checked against any sequence length. Returns
 * ATTN_ERR_BAD_RANGE for negative arguments, q0 + nq or k0 + nk beyond 2^31 - 65, or more
 * than 65535 query blocks of 32.
 */
int attn_dropout_probe(int32_t seq, int32_t head, int32_t q0, int32_t nq, int32_t k0,
                       int32_t nk, float dropout_p, uint64_t seed, uint8_t* keep,
                       void* stream);

/*
 * attn_mask_probe - replays the bf16 forward prefill's mask decisions (its stage range, the
 * per-wave block class of every stage and the per-lane test of the kernel) for query tokens
 * [q0, q0 + nq) against key tokens [k0, k0 + nk) and writes bits[i * nk + j] = 1 if the pair
 * (q0 + i, k0 + j) enters the softmax, else 0 (uint8, device memory, nq * nk bytes). Exists so
 * the mask can be compared bit for bit with an explicit mask built from sequence ids and
 * positions (Causal Mask and Ragged Sequence Layouts, sections 1-4). Same as
 * attn_mask_probe_ex with ATTN_PROBE_PREFILL. Returns ATTN_ERR_BAD_RANGE if the window leaves
 * [0, total_q) x [0, total_k).
 */
int attn_mask_probe(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    int32_t num_seqs, int32_t total_q, int32_t total_k,
                    int32_t mask_mode, int32_t window,
                    int32_t q0, int32_t nq, int32_t k0, int32_t nk,
                    uint8_t* bits, void* stream);

/* Kernel units whose mask decisions attn_mask_probe_ex replays. */
enum attn_probe_unit {
  ATTN_PROBE_PREFILL = 0,          /* bf16 prefill (software-pipelined kernel) */
  ATTN_PROBE_PREFILL_GENERIC = 1,  /* fp32 prefill and every dropout forward */
  ATTN_PROBE_SPLITK = 2,           /* split-K decode: chunk clip + per-lane test, one head */
  ATTN_PROBE_BWD_KV = 3,           /* backward dK / dV kernel (keys on lanes) */
  ATTN_PROBE_BWD_Q = 4,            /* backward dQ kernel (queries on lanes) */
  ATTN_PROBE_BWD_KV_F32 = 5,       /* fp32 backward dK/dV kernel (32-key chunks) */
  ATTN_PROBE_BWD_Q_F32 = 6         /* fp32 backward dQ kernel (32-query chunks) */
};

/*
 * attn_mask_probe_ex - attn_mask_probe for any kernel unit: the unit's own composition of
 * stage ranges, block classes and per-lane tests (the backward's, which rebuild the
 * forward's logical mask: Causal Mask and Ragged Sequence Layouts, section 6), replayed into
 * bits as above. For the backward units a pair counts if it enters the gradient sums (rows
 * past a sequence's end never do). ATTN_PROBE_SPLITK replays the split-K plan attn_fwd_ex
 * chooses for these shapes with num_splits key chunks (0 = the automatic count; bf16,
 * head_dim 128) for query head `head` (the row blocks of a GQA group depend on it); it
 * needs max_seqlen_q/k, Hq and Hkv as for attn_fwd and returns ATTN_ERR_BAD_PLAN where the
 * split-K path does not apply. The other units ignore max_seqlen_q/k, Hq, Hkv, head and
 * num_splits. Errors: ATTN_ERR_BAD_PLAN for an unknown unit, otherwise as attn_mask_probe.
 */
int attn_mask_probe_ex(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int32_t num_seqs, int32_t total_q, int32_t total_k,
                       int32_t max_seqlen_q, int32_t max_seqlen_k,
                       int32_t num_heads_q, int32_t num_heads_kv,
                       int32_t mask_mode, int32_t window, int32_t unit, int32_t head,
                       int32_t num_splits, int32_t q0, int32_t nq, int32_t k0, int32_t nk,
                       uint8_t* bits, void* stream);

/*
 * attn_check_seqlens - checks cu_seqlens_q / cu_seqlens_k on the device against the host
 * sizes the other entry points are given, and writes one int32 to *error_word (device
 * memory, caller-owned; asynchronous on stream): 0 if the arrays are well formed, else the
 * OR of the attn_seqlens_error bits below. The other entry points never read cu_seqlens on
 * the host and treat malformed contents as undefined behaviour; this is the check a caller
 * (or a debug path) runs first. The cumulative-length arrays are what locate each
 * sequence's segment of the packed tensors (Causal Mask and Ragged Sequence Layouts,
 * section 1), and the same arrays must reach the backward (same page, section 6).
 *   reads  cu_seqlens_q[0 .. num_seqs], cu_seqlens_k[0 .. num_seqs] (int32, device)
 *   checks cu[0] == 0, cu[s + 1] >= cu[s], cu[num_seqs] == total, every length <= max_seqlen
 * Errors (nothing is launched): ATTN_ERR_BAD_SHAPE for negative sizes, ATTN_ERR_NULL_PTR for
 * a NULL array or word (num_seqs = 0 still reads cu[0] of both arrays).
 */
enum attn_seqlens_error {
  ATTN_SEQLENS_Q_START = 1,        /* cu_seqlens_q[0] != 0 */
  ATTN_SEQLENS_Q_DECREASING = 2,   /* some cu_seqlens_q[s + 1] < cu_seqlens_q[s] */
  ATTN_SEQLENS_Q_END = 4,          /* cu_seqlens_q[num_seqs] != total_q */
  ATTN_SEQLENS_Q_ABOVE_MAX = 8,    /* some query length > max_seqlen_q */
  ATTN_SEQLENS_K_START = 16,       /* the same four for the keys */
  ATTN_SEQLENS_K_DECREASING = 32,
  ATTN_SEQLENS_K_END = 64,
  ATTN_SEQLENS_K_ABOVE_MAX = 128
};

int attn_check_seqlens(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int32_t num_seqs, int32_t total_q, int32_t total_k,
                       int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t* error_word,
                       void* stream);

/*
 * attn_describe_plan - writes a one-line description of what attn_fwd_ex would launch for
 * these arguments (path, tile shape, split count, grid, workspace, library version) into
 * buf (NUL-terminated, truncated to len). Returns ATTN_OK or a validation error.
 */
int attn_describe_plan(int32_t num_seqs, int32_t total_q, int32_t total_k,
                       int32_t max_seqlen_q, int32_t max_seqlen_k,
                       int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                       int32_t dtype, int32_t mask_mode, int32_t window,
                       int32_t path, int32_t num_splits, char* buf, size_t len);

/* Static description of a status code (never NULL). */
const char* attn_status_string(int status);

/* ATTN_VERSION of the built library. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_TILED_ATTN_H */
