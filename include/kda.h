/*
 * kda.h — C ABI of the MI355X (gfx950) Kimi Delta Attention library (libkda.so).
 *
 * What is computed (per sequence b and head h; heads and sequences are
 * independent).  Sources: "Inside Kimi K3: Architecture of an Open Frontier
 * Model" (academa.ai lecture), sequence paragraph — one state of fixed shape passed
 * from token to token, a per-channel diagonal decay alpha applied to it, then
 * a beta-weighted write that corrects the stored association, with a floor of
 * -5 on the log-decay; "Kimi K3" (meridianbulletin.com), "Handling One Million Tokens
 * with a Fixed-Size State Matrix" (alpha limited to [e^-5, 1]) and
 * "Parallelizing Sequential State Updates" (tokens of a chunk in parallel,
 * then state hand-off; a scheduler that spreads long prefill over the compute
 * units of one card; transitions and increments joined by a prefix scan).
 * The update formula is not printed on the pages; the reading used here, with
 * S a d_k x d_v fp32 matrix whose rows are key channels, is
 *
 *     S <- Diag(exp(clamp(log_alpha_t, -5, 0))) S        forget
 *     S <- S + beta_t k_t (v_t - S^T k_t)^T                delta write
 *     o_t = S^T q_t                                        read after the write
 *
 * No scaling of q or k is applied inside the library; callers pass the
 * (L2-normalised) vectors they want used.  log_alpha values outside [-5, 0]
 * are clamped on load.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains them.  Scratch memory comes only from
 *    the caller's `workspace` (kda_chunk_prefill_noalloc: from a fixed device
 *    array inside the library).
 *  - Layouts are contiguous row-major.  Pointers must be 16-byte aligned
 *    (beta: 4-byte aligned).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; no call synchronises the host with the device.  A split
 *    prefill also uses one stream of the library's own per device (created on
 *    first use, default priority, kept for the life of the process), forked
 *    from and joined back to `stream` by events.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    rejected call returns an error status and enqueues nothing.  A launch
 *    failure returns KDA_ERR_DEVICE.  Valid inputs produce no in-kernel errors.
 *  - No C++ exception crosses this interface.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* bad shape, NULL pointer, misalignment, overlap */
    KDA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (head size, chunk, dtype) */
    KDA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
    KDA_ERR_DEVICE = 4            /* a HIP runtime call or kernel launch failed */
} kda_status_t;

/* Element type of q, k, v and o.  log_alpha, beta and the states are always fp32. */
typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype_t;

/* Returns KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *kda_status_string(kda_status_t status);

/*
 * Sequence-split plan that kda_chunk_prefill picks for a shape (the automatic
 * scheduler): `seg_len` tokens per segment (== T when the sequence is not split;
 * segments of equal length, the last one possibly shorter, few enough that all
 * of them run at once on fewer workgroups than the GPU has compute units) and
 * `n_vs` state-column slices per head.  Pages: "Kimi
 * K3", "Parallelizing Sequential State Updates" (a scheduler spreads
 * long-context prefill over the compute units of one card).  Any output
 * pointer may be NULL.
 */
kda_status_t kda_chunk_prefill_plan(int B, int T, int H, int dk, int dv, int chunk,
                                    kda_dtype_t dtype, int *seg_len, int *n_vs);

/*
 * Bytes of device workspace that kda_chunk_prefill needs (the automatic plan):
 * the per-segment transitions and increments, the segments' entry states and
 * the transition pass's chunk counts of a sequence split, 0 when the sequence
 * is not split.  Returns 0 for shapes that kda_chunk_prefill would reject.
 */
size_t kda_chunk_prefill_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                         kda_dtype_t dtype);

/*
 * kda_chunk_prefill_workspace_bytes for an explicit segment length `seg_len`
 * (0 = the automatic plan), as passed to kda_chunk_prefill_ex.
 */
size_t kda_chunk_prefill_workspace_bytes_ex(int B, int T, int H, int dk, int dv, int chunk,
                                            kda_dtype_t dtype, int seg_len);

/*
 * Chunked KDA prefill over T tokens from the initial state S0.
 * Pages: "Kimi K3", "Parallelizing Sequential State Updates" (chunk-parallel
 * tokens, state hand-off); "Kimi K3's architecture" (orkas.ai), "A lower bound
 * that deleted a GPU code path" (bounded log-decay lets diagonal and
 * off-diagonal 16-token tiles share one dense matrix product).
 *
 *   q, k       [B, T, H, dk]  dtype          queries, keys
 *   v          [B, T, H, dv]  dtype          values
 *   log_alpha  [B, T, H, dk]  fp32           per-channel log forget gate (clamped to [-5, 0])
 *   beta       [B, T, H]      fp32           write strength
 *   S0         [B, H, dk, dv] fp32 or NULL   initial state (NULL = zeros)
 *   o          [B, T, H, dv]  dtype  (out)   outputs o_t = S_t^T q_t
 *   S_T        [B, H, dk, dv] fp32 or NULL   final state (NULL = not written);
 *                                            may be exactly S0 (in place), must not
 *                                            partially overlap it
 *   chunk      16, 32 or 64 tokens per chunk; the result does not depend on it
 *              beyond rounding.  KDA_F32 with chunk 64 runs as 32-token chunks
 *              (fp32 operands of a 64-token chunk exceed the LDS of one workgroup)
 *   dk == dv   64 or 128
 *   workspace  device scratch of at least kda_chunk_prefill_workspace_bytes(...)
 *              bytes (may be NULL when that is 0)
 * T == 0 is valid: S_T receives S0 (or zeros).  B == 0 or H == 0 is a no-op.
 */
kda_status_t kda_chunk_prefill(const void *q, const void *k, const void *v,
                               const float *log_alpha, const float *beta, const float *S0,
                               void *o, float *S_T,
                               int B, int T, int H, int dk, int dv, int chunk,
                               kda_dtype_t dtype, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * kda_chunk_prefill with an explicit plan: `seg_len` tokens per segment (a
 * positive multiple of `chunk`, all segments equal but the last; 0 = automatic;
 * >= T = no split) and `n_vs` state-column slices (1 or 2 for dv = 128, 1 for
 * dv = 64; 0 = automatic).  With a split, segment 0 runs from S0 with its
 * outputs; the transitions M_s of the later segments (the recurrence applied to
 * the identity with zero values) are formed only until every entry has fallen
 * below 2^-126, and are then stored as zeros; segments 1 .. n-1 run with their
 * outputs from a zero state, which gives the increments H_s; an on-device
 * prefix scan S_in(s+1) = M_s S_in(s) + H_s from segment 0's final state gives
 * every later entry state; and each segment reruns from its entry state only
 * the chunks before its transition died, overwriting those outputs (all of
 * them where the transition never dies, e.g. with no decay and beta = 0).  Past
 * that point an entry state adds less than dk * 2^-126 times its own size to
 * the state, so the results are those of one pass up to rounding.  Segment 0
 * runs on a second stream of the library (created once per device, default
 * priority) joined back to `stream` by events (fork after the work already on
 * `stream`, join before the scan); the call stays asynchronous.  Calls from
 * several host threads are serialised while they enqueue a split.
 * Pages: "Kimi K3's architecture", "The bill comes due in the serving stack"
 * (per segment, the transition and the state reached from zero combine
 * exactly across segments); "Inside Kimi K3" (academa.ai lecture), sequence
 * paragraph (the diagonal gate scales down what the state keeps from earlier
 * tokens).
 * The workspace must hold kda_chunk_prefill_workspace_bytes_ex(..., seg_len).
 */
kda_status_t kda_chunk_prefill_ex(const void *q, const void *k, const void *v,
                                  const float *log_alpha, const float *beta, const float *S0,
                                  void *o, float *S_T,
                                  int B, int T, int H, int dk, int dv, int chunk,
                                  kda_dtype_t dtype, int seg_len, int n_vs,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_chunk_prefill_ex that also checkpoints the state for prefix reuse: S_ckpt[b, i] is the
 * state after the first (i + 1) * ckpt_every tokens of sequence b, for i < T / ckpt_every.
 * Pages: "Kimi K3's architecture" (orkas.ai), "The bill comes due in the serving stack" (a
 * prefix-cache hit needs the recurrent state restorable at the same boundary as the token
 * pages; the state is checkpointed only at a sparse subset of the 512-token hash endpoints,
 * e.g. ckpt_every = 4096).
 *
 *   ckpt_every  0 (no checkpoints: identical to kda_chunk_prefill_ex) or a positive multiple
 *               of `chunk`
 *   S_ckpt      [B, T / ckpt_every, H, dk, dv] fp32, written only; must not overlap any other
 *               argument (may be NULL when T < ckpt_every)
 * Other arguments, plans, workspace and errors as for kda_chunk_prefill_ex.
 */
kda_status_t kda_chunk_prefill_ckpt(const void *q, const void *k, const void *v,
                                    const float *log_alpha, const float *beta, const float *S0,
                                    void *o, float *S_T,
                                    int B, int T, int H, int dk, int dv, int chunk,
                                    kda_dtype_t dtype, int ckpt_every, float *S_ckpt,
                                    int seg_len, int n_vs,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_chunk_prefill_ex with the bounded gate fused: the decay input is the raw gate
 * pre-activation x (bf16) and log alpha = -5 * sigmoid(x) is formed on load, which moves 2
 * instead of 4 bytes per key channel and token.  Pages: "Inside Kimi K3" (academa.ai lecture),
 * sequence paragraph (the decay curve itself is changed so that it is bounded below at -5);
 * "Kimi K3's architecture" (orkas.ai), "A lower bound that deleted a GPU code path" (the
 * activation has to be bounded below).  The pages do not print the curve; -5 * sigmoid is the
 * reading used, the one the benchmark workloads draw log alpha from.
 *
 *   gate       [B, T, H, dk]  bf16   raw gate pre-activation (in place of log_alpha)
 * Other arguments, plans, workspace and errors as for kda_chunk_prefill_ex.  Supported for
 * dtype KDA_BF16 with dk == dv == 128 (one column slice; n_vs must be 0 or 1); other shapes
 * return KDA_ERR_UNSUPPORTED.
 */
kda_status_t kda_chunk_prefill_gate(const void *q, const void *k, const void *v,
                                    const void *gate, const float *beta, const float *S0,
                                    void *o, float *S_T,
                                    int B, int T, int H, int dk, int dv, int chunk,
                                    kda_dtype_t dtype, int seg_len, int n_vs,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step for N independent sequences: exactly one token of the
 * recurrence, with the state read and written in place.  Pages: "Inside Kimi
 * K3", sequence paragraph (constant cost per new token); "Kimi K3's
 * architecture", "The bill comes due in the serving stack" (the state updates
 * in place).
 *
 *   q, k       [N, H, dk]      dtype
 *   v          [N, H, dv]      dtype
 *   log_alpha  [N, H, dk]      fp32   (clamped to [-5, 0])
 *   beta       [N, H]          fp32
 *   S          [N, H, dk, dv]  fp32   in/out, updated in place
 *   o          [N, H, dv]      dtype  (out)
 *   dk == dv   64 or 128
 * N == 0 or H == 0 is a no-op.  o must not overlap any input or S.
 */
kda_status_t kda_decode_step(const void *q, const void *k, const void *v,
                             const float *log_alpha, const float *beta, float *S, void *o,
                             int N, int H, int dk, int dv, kda_dtype_t dtype, void *stream);

/*
 * Speculative decoding, verify step: m >= 1 drafted tokens per sequence, run from the current
 * state S, with the outputs of all m tokens written to o and S left unchanged.  Pages: "Kimi
 * K3's architecture" (orkas.ai), "The bill comes due in the serving stack" (the state is
 * updated in place, so a rejected draft cannot be undone; the projected inputs are kept and
 * the state is rebuilt on chip).  Blocks of up to 16 tokens run as a token loop with the state
 * held on chip (read once); longer blocks, of any length m, run as one unsplit chunked prefill
 * over the block (chunk 32 or 64, one workgroup per sequence and head; no workspace needed).
 *
 *   q, k       [N, m, H, dk]  dtype          drafted queries, keys
 *   v          [N, m, H, dv]  dtype
 *   log_alpha  [N, m, H, dk]  fp32           (clamped to [-5, 0])
 *   beta       [N, m, H]      fp32
 *   S          [N, H, dk, dv] fp32           state before the block (read only)
 *   o          [N, m, H, dv]  dtype  (out)   o[n, t] = S_t^T q_t for t < m
 *   dk == dv   64 or 128
 * N == 0 or H == 0 is a no-op.  Errors as for kda_chunk_prefill.
 */
kda_status_t kda_spec_verify(const void *q, const void *k, const void *v,
                             const float *log_alpha, const float *beta, const float *S,
                             void *o, int N, int m, int H, int dk, int dv, kda_dtype_t dtype,
                             void *stream);

/*
 * Speculative decoding, commit step: advance S in place over the first accepted[n] of the m
 * cached drafted tokens of sequence n (the same inputs given to kda_spec_verify), rebuilding
 * the state from those inputs instead of rolling it back.  Same source as kda_spec_verify.
 *
 *   q, k, v, log_alpha, beta   as for kda_spec_verify
 *   S          [N, H, dk, dv] fp32  in/out   state before the block on entry, state after the
 *                                            accepted tokens on return
 *   accepted   [N]            int32 DEVICE   tokens to keep per sequence; values outside
 *                                            [0, m] are clamped on the device (0 leaves S as is)
 * No output rows are written.  S must not overlap any input.  N == 0 or H == 0 is a no-op.
 * Blocks longer than 16 tokens, of any length m, run as one unsplit chunked prefill with
 * per-sequence lengths (no workspace needed).
 */
kda_status_t kda_spec_commit(const void *q, const void *k, const void *v,
                             const float *log_alpha, const float *beta, float *S,
                             const int *accepted, int N, int m, int H, int dk, int dv,
                             kda_dtype_t dtype, void *stream);

/*
 * Largest workspace kda_chunk_prefill_noalloc can serve: the bytes of the device
 * array it uses in place of a caller workspace (one per GPU the library runs on,
 * held until the process ends).  64 MiB covers, for example, a 1M-token sequence
 * of 16 heads at d = 128 split into 17 segments (49 MiB).
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * kda_chunk_prefill_ex for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument, and no call to hipMalloc, hipFree or any
 * other allocating routine.  A sequence split takes its transitions, increments
 * and entry states from a fixed device array of KDA_NOALLOC_SCRATCH_BYTES bytes
 * inside the library, and every one of its launches runs on `stream` (segment 0
 * inside the zero-start launch of the other segments, not on a second stream).
 *
 *   arguments as for kda_chunk_prefill_ex, without workspace / workspace_bytes
 *   returns KDA_ERR_WORKSPACE when kda_chunk_prefill_workspace_bytes_ex(..., seg_len)
 *   exceeds KDA_NOALLOC_SCRATCH_BYTES (choose a longer seg_len, or call
 *   kda_chunk_prefill_ex with a workspace); other errors as for kda_chunk_prefill_ex.
 *
 * All calls on one GPU share that GPU's array, and it keeps the last call's contents (every
 * byte a call reads was written earlier by the same call).  Calls that overlap on one GPU —
 * enqueued on different streams with no ordering between them, or from several host threads
 * at once — race on it; callers serialise them.
 */
kda_status_t kda_chunk_prefill_noalloc(const void *q, const void *k, const void *v,
                                       const float *log_alpha, const float *beta, const float *S0,
                                       void *o, float *S_T,
                                       int B, int T, int H, int dk, int dv, int chunk,
                                       kda_dtype_t dtype, int seg_len, int n_vs, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
