/*
 * kda.h - C ABI of the MI355X (gfx950) Kimi Delta Attention forward operator.
 *
 * The operator is the channel-wise gated delta rule
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * ("Kimi Linear: An Expressive, Efficient Attention Architecture",
 * paper-graph-ui review, section "The KDA State Update Equation"; Eq. 1 of
 * the "L2 Deep Distill" page). Prefill uses the chunkwise WY/UT algorithm of
 * the review's section "Chunkwise Parallelization" (UT transform, Eq. 8
 * state update, Eq. 9 output) with chunks of KDA_CHUNK tokens; decode is one
 * step of the recurrence per sequence (the review's "FLOPs Accounting and
 * Inference Strategy": chunk kernel for prefill, recurrent kernel for
 * generation).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    never allocates device memory; scratch space is a caller-supplied
 *    workspace sized by kda_chunk_fwd_workspace_bytes() (or, for
 *    kda_chunk_fwd_noalloc, a fixed array inside the library).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream). Nothing synchronises the host.
 *  - Arguments that the host can see (pointers, sizes, dtypes, aliasing) are
 *    checked before anything is launched; a failed check returns a status
 *    and launches nothing. A launch failure returns KDA_ERR_HIP. No C++
 *    exception crosses the ABI.
 *  - Only d_k = d_v = 128 is supported (the pages' head size).
 *  - Tensor pointers are 16-byte aligned (beta and cu_seqlens: 4-byte), as
 *    every torch allocation is; the kernels move 16-byte vectors. A
 *    misaligned pointer returns KDA_ERR_ALIGN and launches nothing.
 *  - Tensor layouts are dense row-major with the last index fastest:
 *      q, k       [T, H, d_k]   I/O dtype
 *      v, o       [T, H, d_v]   I/O dtype
 *      log_alpha  [T, H, d_k]   float32: natural log of the per-channel decay
 *                               alpha_t in (0, 1], i.e. finite and <= 0
 *      beta       [T, H]        float32
 *      states     [N, H, d_k, d_v] float32 (kda_recurrent_fwd also takes
 *                               bfloat16), S[c][j]: row c = key channel,
 *                               column j = value channel
 *    For decode, T is replaced by the batch N (one token per sequence).
 *  - No query scaling is applied (o_t = S_t^T q_t as printed), q and k are
 *    used as given unless KDA_FLAG_QK_L2NORM asks the kernel to normalise
 *    them, and bf16 outputs are rounded to nearest even.
 *  - Unchecked preconditions (the device cannot report them synchronously):
 *    finite inputs, log_alpha <= 0, cu_seqlens non-decreasing with
 *    cu_seqlens[0] = 0 and cu_seqlens[N] = T. Violations give unspecified
 *    values but never out-of-bounds accesses: kernels clamp every index, and
 *    a malformed cu_seqlens sets the workspace status word (below).
 *    kda_check_inputs() checks all of them on request.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_CHUNK 64    /* tokens per chunk of the chunkwise algorithm */
#define KDA_HEAD_DIM 128 /* the only supported d_k = d_v */

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL                   */
  KDA_ERR_SHAPE = 2,       /* a size is negative or inconsistent           */
  KDA_ERR_UNSUPPORTED = 3, /* d_k or d_v != 128, or unknown dtype          */
  KDA_ERR_WORKSPACE = 4,   /* workspace missing, too small or misaligned   */
  KDA_ERR_ALIAS = 5,       /* an output overlaps an input it must not      */
  KDA_ERR_HIP = 6,         /* the HIP runtime reported a launch error      */
  KDA_ERR_ALIGN = 7,       /* a tensor pointer is misaligned (see above)   */
  KDA_ERR_SCRATCH = 8      /* the call needs more workspace than
                              kda_chunk_fwd_noalloc's fixed array holds    */
} kda_status;

typedef enum {
  KDA_IO_F32 = 0,  /* q, k, v, o are float32 */
  KDA_IO_BF16 = 1  /* q, k, v, o are bfloat16 */
} kda_io_dtype;

/* Flag bits of kda_chunk_fwd and kda_recurrent_fwd. KDA_FLAG_QK_L2NORM
 * replaces q_t and k_t by x / sqrt(sum_c x_c^2 + 1e-6) before use: the
 * pages' L2Norm of queries and keys (review section "Neural
 * Parameterization"), fused into the operator as the "L2 Deep Distill"
 * page's serving note does. The pages give no epsilon; 1e-6 keeps zero
 * vectors at zero. Unknown bits are rejected with KDA_ERR_UNSUPPORTED. */
#define KDA_FLAG_QK_L2NORM 1u
/* Flag bit of kda_chunk_fwd (and its _phase and _noalloc forms):
 * KDA_FLAG_STATE_BF16 makes h0 and h_final bfloat16 [N, H, 128, 128], the
 * state format of the "L2 Deep Distill" page's serving notes (32 x 128 x
 * 128 bf16, 1 MB per layer), which kda_recurrent_fwd also takes
 * (KDA_STATE_BF16). The call widens h0 to float32, carries the state in
 * float32 across all of a sequence's chunks (and windows) and rounds it to
 * bf16 (nearest even) once, into h_final. */
#define KDA_FLAG_STATE_BF16 2u

/*
 * kda_chunk_fwd_workspace_bytes, kda_chunk_fwd_workspace_min_bytes
 *   Recommended and smallest sizes of the device workspace of kda_chunk_fwd
 *   for these sizes (0 if an argument is invalid). The workspace must be
 *   256-byte aligned.
 *   n_seqs: sequences N in the packed batch (N = 1 when cu_seqlens is NULL).
 *   total_tokens: T, tokens over all sequences.
 *   The prefill runs over windows of chunk slots, as many slots per window
 *   as the given workspace holds (below), so any size from the smallest up
 *   works and the results do not depend on it. For one sequence the
 *   recommended size holds every chunk of calls up to about 512 MiB of
 *   intermediates in bf16, 1 GiB in float32 (8192 tokens x 32 heads is one
 *   window either way) and that much otherwise: it does not grow with T
 *   beyond that. Windows follow the
 *   chunk slots in sequence order, so a window holds few sequences of a
 *   packed batch and windows run one after the other: for N > 1 the
 *   recommended size holds up to 8 GiB of intermediates. The smallest size
 *   holds one chunk slot (slowest).
 */
size_t kda_chunk_fwd_workspace_bytes(int32_t n_seqs, int64_t total_tokens,
                                     int32_t heads, int32_t dk, int32_t dv,
                                     kda_io_dtype io);
size_t kda_chunk_fwd_workspace_min_bytes(int32_t n_seqs, int64_t total_tokens,
                                         int32_t heads, int32_t dk, int32_t dv,
                                         kda_io_dtype io);

/*
 * kda_chunk_fwd - chunked prefill over a packed batch of sequences.
 *
 * Computes, for every sequence n (tokens [cu_seqlens[n], cu_seqlens[n+1]))
 * and head h independently, the outputs o_t of every token and the state
 * after the last token, starting from h0[n, h] (zeros when h0 is NULL).
 * Chunks of KDA_CHUNK tokens never straddle sequences; a sequence's last
 * chunk may be shorter. Paper: review section "Chunkwise Parallelization",
 * Eq. 8 (chunk state update) and Eq. 9 (chunk output); the UT transform
 * gives W and U from StrictTril(Diag(beta)(Gamma*K)(K/Gamma)^T).
 *
 *   q, k, v, o      see layouts above; io selects float32 or bfloat16
 *   log_alpha, beta float32
 *   flags           KDA_FLAG_QK_L2NORM (q, k normalised in the kernel) and
 *                   KDA_FLAG_STATE_BF16 (h0, h_final in bfloat16), or 0
 *   h0              [N, H, 128, 128] float32 (bfloat16 with
 *                   KDA_FLAG_STATE_BF16), or NULL for zero states
 *   cu_seqlens      device int32 [N + 1], or NULL for one sequence (N = 1)
 *   h_final         [N, H, 128, 128] in h0's type, or NULL to skip; it may be the
 *                   same pointer as h0 (in-place continuation) but must not
 *                   partially overlap it
 *   workspace       device scratch of at least
 *                   kda_chunk_fwd_workspace_min_bytes(...) bytes (the
 *                   recommended size is kda_chunk_fwd_workspace_bytes(...)),
 *                   256-byte aligned; its contents on return are described
 *                   below
 *   A sequence of length 0 copies h0 (or zeros) to h_final. T = 0 writes
 *   nothing but h_final.
 *   Errors: KDA_ERR_NULL (q, k, v, log_alpha, beta or o NULL when T > 0;
 *   cu_seqlens NULL with n_seqs != 1), KDA_ERR_SHAPE (negative sizes,
 *   n_seqs < 1, heads < 1, T > INT32_MAX with cu_seqlens, more than 2^27
 *   (sequence, head) pairs),
 *   KDA_ERR_UNSUPPORTED (d_k, d_v != 128, unknown dtype or flag bit,
 *   heads > 65535),
 *   KDA_ERR_WORKSPACE (NULL, smaller than the minimum, not 256-byte
 *   aligned),
 *   KDA_ERR_ALIAS (o overlapping an input; h_final overlapping q, k, v,
 *   log_alpha, beta or o; h_final partially overlapping h0), KDA_ERR_HIP.
 *
 * Workspace contents after the call (for inspection and tests; the format
 * is internal and may change). E is the element type: bf16 for
 * KDA_IO_BF16, float32 for KDA_IO_F32. The chunk slots 0 .. S - 1, with
 * S = ceil(T / 64) + N - 1 (at least the chunk count), run in windows of
 * W slots, W = min(S, (bytes - inter_offset) / (H * block)): per window
 * the intra-chunk kernel fills the window's blocks, then the carry
 * consumes them.
 *   [0, 4)          int32 status: 0 ok, 1 malformed cu_seqlens
 *   [256, ...)      int32 chunk_offset[N + 1]: first global chunk index of
 *                   each sequence (exclusive prefix sum of ceil(L_n / 64))
 *   [state_offset)  two float32 [H, 128, 128] states, state_offset =
 *                   256 + round_up(4 (N + 1), 256): the state of the
 *                   sequence crossing a window boundary, left by one window
 *                   for the next (the two slots alternate)
 *   [inter_offset)  per (chunk b of the last window, head h), a block of
 *                   block = 40960 E + 128 float32 bytes, ordered
 *                   [b - W0][h] (W0 = the window's first slot), where
 *                   inter_offset = state_offset + 2 * H * 65536:
 *       XA  16384 E  [-W ; Qt]  as A-fragments, 8 row tiles x 4 k-blocks
 *       KT   8192 E  K'^T       as A-fragments, 8 row tiles x 2 k-blocks
 *       UC  16384 E  U and Ut^T as C-fragments, 8 column tiles x 8 row
 *                    tiles: row tiles 0-3 hold U (rows = token), 4-7 hold
 *                    Ut^T (rows = value column)
 *       GC   128 f32 gamma_C[c] = exp(g_last[c])
 *   with, inside the chunk (rows i = token position, padded to 64 with
 *   k = v = q = 0, beta = 0, log_alpha = 0):
 *       g_i   = sum_{t <= i} log_alpha_t,        Gamma rows exp(g_i)
 *       L     = StrictTril(Diag(beta) A_kk),     A_kk[i][t] = sum_c k_i k_t exp(g_i - g_t)
 *       W     = (I + L)^{-1} Diag(beta) (Gamma * K),  U = (I + L)^{-1} Diag(beta) V
 *       A_qk  = Tril(sum_c q_i k_t exp(g_i - g_t))
 *       Qt    = Gamma * Q - A_qk W,  Ut = A_qk U,  K'[t][c] = k_t[c] exp(g_last[c] - g_t[c])
 *   so that, from the chunk's start state S, U - W S is the pseudo-value,
 *   O = Qt S + Ut (Eq. 9 regrouped; computed transposed, O^T = Ut^T +
 *   S^T Qt^T) and the next state is Diag(gamma_C) S + K'^T (U - W S)
 *   (Eq. 8).
 *   Fragment maps: an A-fragment (mt, kb) of matrix X gives lane
 *   l = r + 16 g (r < 16, g < 4) the 8 elements X[16 mt + r][32 kb + 4 g + e]
 *   for e < 4 and X[16 mt + r][32 kb + 16 + 4 g + e - 4] for e >= 4; a
 *   C-fragment (jt, mt) gives lane l the 4 elements U[16 mt + 4 g + e][16 jt + r]
 *   for mt < 4 and Ut[16 (mt - 4) + r][16 jt + 4 g + e] for mt >= 4.
 *   Fragments are stored lane-major, A-fragments ordered [mt][kb],
 *   C-fragments ordered [jt][mt].
 */
kda_status kda_chunk_fwd(const void *q, const void *k, const void *v,
                         const float *log_alpha, const float *beta,
                         const void *h0, const int32_t *cu_seqlens,
                         int32_t n_seqs, int64_t total_tokens, int32_t heads,
                         int32_t dk, int32_t dv, kda_io_dtype io,
                         uint32_t flags, void *o, void *h_final,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * kda_chunk_fwd_phase - one of the three launches that make up kda_chunk_fwd,
 * for per-kernel timing and inspection of the workspace.
 *   phase 0: chunk map (chunk_offset and status from cu_seqlens)
 *   phase 1: intra-chunk kernel (gate cumsum, UT transform; fills the
 *            per-chunk blocks of the workspace)
 *   phase 2: carry kernel (state propagation and chunk outputs; writes o and
 *            h_final)
 * Arguments, validation and errors are those of kda_chunk_fwd (an invalid
 * phase returns KDA_ERR_SHAPE), except that the workspace must hold every
 * chunk slot in one window (else KDA_ERR_WORKSPACE). Phases 0, 1, 2
 * enqueued in order on one stream with the same arguments compute exactly
 * what kda_chunk_fwd does.
 */
kda_status kda_chunk_fwd_phase(int32_t phase, const void *q, const void *k,
                               const void *v, const float *log_alpha,
                               const float *beta, const void *h0,
                               const int32_t *cu_seqlens, int32_t n_seqs,
                               int64_t total_tokens, int32_t heads, int32_t dk,
                               int32_t dv, kda_io_dtype io, uint32_t flags,
                               void *o, void *h_final, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * kda_chunk_fwd_noalloc - kda_chunk_fwd without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * The workspace is a fixed array of KDA_NOALLOC_SCRATCH_BYTES bytes of
 * device memory inside the library, one per GPU, held from the first call
 * on that GPU until the process ends; the call uses the copy of the calling
 * thread's current device (the stream must belong to it). The call
 * allocates nothing (no hipMalloc, no library allocation); the caller still
 * supplies every input and output. Arguments, results and errors are those
 * of kda_chunk_fwd, plus KDA_ERR_SCRATCH when
 * kda_chunk_fwd_workspace_min_bytes(...) for these sizes exceeds the array
 * (returned before any HIP call) and KDA_ERR_HIP when the array's device
 * address cannot be obtained. The prefill's windows are sized to the array
 * (about 50 chunk slots at 32 bf16 heads), so T is not limited by it. Every call on one GPU uses the same array and
 * leaves its contents behind (the workspace contents kda_chunk_fwd
 * describes): calls that overlap on one GPU, on different streams or from
 * different threads, race and give undefined results; calls ordered on one
 * stream do not.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (128u << 20) /* 128 MiB per GPU */
kda_status kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                 const float *log_alpha, const float *beta,
                                 const void *h0, const int32_t *cu_seqlens,
                                 int32_t n_seqs, int64_t total_tokens,
                                 int32_t heads, int32_t dk, int32_t dv,
                                 kda_io_dtype io, uint32_t flags, void *o,
                                 void *h_final, void *stream);

/*
 * kda_decode_step - one recurrent step for a batch of sequences.
 *
 * For each sequence n and head h, with alpha = exp(log_alpha[n, h]):
 *   S~ = Diag(alpha) S,  e = S~^T k,  S <- S~ - beta k (e - v)^T,
 *   o  = S^T q (on the updated state)
 * which is Eq. 1 written in the review's "Online Learning Interpretation"
 * form (decode = "the recurrent kernel (Eq. 2)" of the review's "FLOPs
 * Accounting and Inference Strategy"). S_inout [N, H, 128, 128] float32 is
 * read once and overwritten in place.
 *   q, k [N, H, 128], v [N, H, 128], o [N, H, 128]: I/O dtype
 *   log_alpha [N, H, 128], beta [N, H]: float32
 * It is kda_recurrent_fwd with one token per sequence, an fp32 state
 * updated in place and no flags (same kernel, same results).
 * n_seqs = 0 does nothing. Errors: KDA_ERR_NULL, KDA_ERR_SHAPE (negative
 * sizes, heads < 1, more than 2^29 (sequence, head) pairs),
 * KDA_ERR_UNSUPPORTED, KDA_ERR_ALIAS (S_inout or o overlapping an input, or
 * each other), KDA_ERR_HIP.
 */
kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           float *S_inout, int32_t n_seqs, int32_t heads,
                           int32_t dk, int32_t dv, kda_io_dtype io, void *o,
                           void *stream);

typedef enum {
  KDA_STATE_F32 = 0,  /* recurrent states are float32 */
  KDA_STATE_BF16 = 1  /* recurrent states are bfloat16 (rounded to nearest even) */
} kda_state_dtype;

/*
 * kda_recurrent_fwd - fused token-by-token forward over a packed batch.
 *
 * Computes exactly what kda_chunk_fwd computes (outputs o_t of every token and
 * the state after each sequence's last token, from h0 or zeros), but runs the
 * recurrence one token at a time with each state held on chip for the whole
 * sequence: the state is read once and written once per call, whatever the
 * sequence length. This is the recurrent kernel the review's "FLOPs
 * Accounting and Inference Strategy" section gives generation, and the one
 * the "L2 Deep Distill" page's serving note selects for inputs of at most 64
 * new tokens per sequence (multi-token decode, speculative verification).
 * Any length works; beyond a few dozen tokens kda_chunk_fwd is faster.
 * Per token, with alpha = exp(log_alpha):
 *   S~ = Diag(alpha) S,  e = S~^T k,  S <- S~ + beta k (v - e)^T,  o = S^T q.
 *
 *   q, k, v, o, log_alpha, beta  layouts as for kda_chunk_fwd ([T, H, 128],
 *                   beta [T, H]); io selects float32 or bfloat16 q, k, v, o
 *   h0, h_final     [N, H, 128, 128] in state_dtype; h0 NULL means zero
 *                   states, h_final NULL skips the write; h_final may be the
 *                   same pointer as h0 (in-place update, the decode case) but
 *                   must not partially overlap it
 *   cu_seqlens      device int32 [N + 1], or NULL: then every sequence has
 *                   total_tokens / n_seqs tokens (q is [N, L, H, 128]) and
 *                   total_tokens must be a multiple of n_seqs
 *   state_dtype     KDA_STATE_F32, or KDA_STATE_BF16: states are widened to
 *                   float32 on chip, so a call over L tokens rounds the state
 *                   once, not L times (the pages' serving note keeps the
 *                   state in BF16, 1 MB per layer)
 *   flags           0 or KDA_FLAG_QK_L2NORM (q, k normalised in the kernel)
 *   n_seqs = 0 (with total_tokens = 0) does nothing. A sequence of length 0
 *   copies h0 (or zeros) to h_final.
 *   Errors: KDA_ERR_NULL (q, k, v, log_alpha, beta or o NULL when T > 0),
 *   KDA_ERR_SHAPE (negative sizes, heads < 1, n_seqs = 0 with T > 0,
 *   T not a multiple of n_seqs without cu_seqlens, T > INT32_MAX with
 *   cu_seqlens, more than 2^29 (sequence, head) pairs),
 *   KDA_ERR_UNSUPPORTED (d_k, d_v != 128, unknown dtype or flag bit),
 *   KDA_ERR_ALIAS (o overlapping an input or h_final; h_final overlapping q,
 *   k, v, log_alpha, beta, cu_seqlens; h_final partially overlapping h0),
 *   KDA_ERR_HIP. With cu_seqlens, values outside [0, T] or decreasing are
 *   clamped (unspecified results, no out-of-bounds access).
 */
kda_status kda_recurrent_fwd(const void *q, const void *k, const void *v,
                             const float *log_alpha, const float *beta,
                             const void *h0, const int32_t *cu_seqlens,
                             int32_t n_seqs, int64_t total_tokens,
                             int32_t heads, int32_t dk, int32_t dv,
                             kda_io_dtype io, kda_state_dtype state_dtype,
                             uint32_t flags, void *o, void *h_final,
                             void *stream);

/*
 * kda_rmsnorm_gate - the output epilogue: head-wise RMSNorm times a sigmoid
 * gate (FusedRMSNormGated).
 *
 * For every row r (one token of one head) of d_v = 128 channels:
 *   y[r][j] = sigmoid(gate[r][j]) * o[r][j] / sqrt(mean_j o[r][j]^2 + eps)
 *             * weight[j]
 * Paper: "Kimi Linear" review, section "Neural Parameterization", output
 * gate equation (a head-wise RMSNorm of the operator's output and a
 * data-dependent sigmoid gate before the output projection); the "L2 Deep
 * Distill" page's module list fuses the two. The pages give no eps and no
 * form for the norm's weight: here eps is the caller's, and the weight is
 * one vector of 128 entries shared by all heads, or NULL for ones.
 *
 *   o, gate, y  [rows, 128] in the I/O dtype; o is kda_chunk_fwd's or
 *               kda_recurrent_fwd's output viewed as [T * H, 128], gate the
 *               gate pre-activation in the same layout
 *   weight      [128] float32, or NULL
 *   eps         finite, >= 0
 *   y may be the same pointer as o (in place) but must not partially
 *   overlap it, nor overlap gate or weight. rows = 0 does nothing.
 *   Errors: KDA_ERR_NULL (o, gate or y NULL with rows > 0), KDA_ERR_SHAPE
 *   (rows < 0 or > 2^36, eps negative, NaN or infinite),
 *   KDA_ERR_UNSUPPORTED (dv != 128, unknown dtype), KDA_ERR_ALIAS,
 *   KDA_ERR_HIP.
 */
kda_status kda_rmsnorm_gate(const void *o, const void *gate,
                            const float *weight, float eps, int64_t rows,
                            int32_t dv, kda_io_dtype io, void *y,
                            void *stream);

/*
 * kda_check_inputs - debug check of the preconditions the compute entry
 * points document but cannot verify on the device.
 *
 * The gate is the natural log of a per-channel decay alpha in (0, 1] (the
 * "Kimi Linear" review, section "The KDA State Update Equation", gives a
 * decay per key channel in [0, 1]; alpha = 0 has no finite log), so every
 * log_alpha element must be finite and <= 0; q, k, v and beta must be
 * finite; a packed batch needs 0 = cu_seqlens[0] <= ... <= cu_seqlens[N] = T.
 * The call reads the inputs once (the same tensors and layout as
 * kda_chunk_fwd, or the decode step's with T = N) and writes to *flags, on
 * the device and asynchronously on `stream`, the OR of
 *   KDA_BAD_QKV   a non-finite element of q, k or v
 *   KDA_BAD_GATE  a log_alpha element that is NaN, +-inf or > 0
 *   KDA_BAD_BETA  a non-finite beta
 *   KDA_BAD_CU    cu_seqlens not rising from 0 to T (only if cu_seqlens is
 *                 not NULL; n_seqs is ignored when it is NULL)
 * so 0 means every documented precondition holds. flags is one int32 of
 * device memory owned by the caller (4-byte aligned), written by a kernel
 * (no memset: the call may be captured in a HIP graph).
 * Errors: KDA_ERR_NULL (flags NULL, or a tensor NULL with T > 0),
 * KDA_ERR_SHAPE (T < 0, heads < 1, n_seqs < 1 with cu_seqlens, T * heads
 * above 2^40), KDA_ERR_UNSUPPORTED (dk or dv != 128, unknown dtype, heads
 * > 65535), KDA_ERR_ALIGN, KDA_ERR_ALIAS (flags inside an input),
 * KDA_ERR_HIP.
 */
#define KDA_BAD_QKV 1
#define KDA_BAD_GATE 2
#define KDA_BAD_BETA 4
#define KDA_BAD_CU 8
kda_status kda_check_inputs(const void *q, const void *k, const void *v,
                            const float *log_alpha, const float *beta,
                            const int32_t *cu_seqlens, int32_t n_seqs,
                            int64_t total_tokens, int32_t heads, int32_t dk,
                            int32_t dv, kda_io_dtype io, int32_t *flags,
                            void *stream);

/* Static description of a status code (never NULL). */
const char *kda_status_string(kda_status s);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
