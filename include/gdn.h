/*
 * gdn.h -- libgdn: gated delta-rule linear attention (Gated DeltaNet) on one
 * AMD Instinct MI355X (gfx950).  Plain C ABI: device pointers, sizes, a HIP
 * stream handle and an int status.  No allocation, no synchronisation.
 *
 * The operation (Qwen3.5-9B-npu model page, "How it works" -> "Gated DeltaNet
 * on the NPU"): per head, a state S of dk x dv (row index over the key
 * dimension, column index over the value dimension) is carried through the
 * tokens of a sequence; for token t
 *
 *     S   <- S * exp(g_t)
 *     kv  <- S^T k_t
 *     S   <- S + k_t (outer) ((v_t - kv) * beta_t)
 *     o_t <- S^T q_t
 *
 * No 1/sqrt(dk) scale and no normalisation of q or k is applied inside: the
 * caller passes q and k as they should enter the recurrence.
 *
 * Conventions shared by both calls
 *   - Shapes: dk == dv == 128 (the page's per-head state is 128 x 128); other
 *     sizes return GDN_ERR_UNSUPPORTED.
 *   - dtypes: q, k, v and the outputs O/o share io_dtype (GDN_F32 or GDN_BF16);
 *     g, beta and the states are always fp32.  Outputs in bf16 are rounded to
 *     nearest even from fp32.
 *   - Layout: every tensor is dense and row-major in the shape given; base
 *     pointers of q, k, v, O/o and the states must be 16-byte aligned, g and
 *     beta 4-byte aligned.
 *   - Ownership: every pointer is caller-owned device memory.  The library
 *     allocates nothing, keeps no state between calls and never waits on the
 *     device, so a call may be captured into a HIP graph.
 *   - Streams: work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and the call returns at once.  Faults inside a kernel surface at
 *     the caller's next synchronisation.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; a rejected call enqueues nothing.  A failed launch returns
 *     GDN_ERR_HIP.
 *   - Preconditions not checked: g <= 0 and 0 <= beta <= 1 (the accuracy
 *     contract assumes them), finite inputs (NaN/Inf propagate).  For bf16
 *     io the prompt form's matrix operands are fp16 (q and k, split pairs
 *     where the recurrence needs them) and bf16 (v): q and k must have
 *     entries of unit scale (|x| well below 6.5e4 / 128, as L2-normalised
 *     rows, or up to the page's q x 1024 rescale); v and the states may have
 *     any magnitude from about 2^-55 to 2^55 (each head's values are held at
 *     a power-of-two scale inside the kernel).
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1,   /* NULL pointer, negative size, misalignment */
    GDN_ERR_UNSUPPORTED = 2,   /* dk/dv != 128, chunk not in {16,32,64}, dtype */
    GDN_ERR_ALIAS = 3,         /* buffers overlap in a way the call forbids */
    GDN_ERR_HIP = 4,           /* the HIP runtime refused the launch */
    GDN_ERR_SCRATCH = 5        /* more scratch than gdn_chunk_prefill_segmented_noalloc holds */
} gdn_status;

typedef enum {
    GDN_F32 = 0,
    GDN_BF16 = 1,
    /* bf16 q, k, v with an fp32 O: the arithmetic of the bf16 path without the
     * rounding of O to bf16.  Accepted by gdn_chunk_prefill and
     * gdn_chunk_prefill_ex only (O is then [B, T, H, 128] fp32). */
    GDN_BF16_F32_OUT = 2
} gdn_dtype;

/* How the prompt form's matrix-core kernel forms the 16 x 16 diagonal blocks of
 * (I + N)^-1 (see gdn_chunk_prefill_ex). */
typedef enum {
    GDN_INVERSE_DEFAULT = 0,        /* the library's choice */
    GDN_INVERSE_SUBSTITUTION = 1,   /* back substitution, fp32, on the vector ALUs */
    GDN_INVERSE_DOUBLING = 2        /* exact block doubling on the matrix cores */
} gdn_inverse;

/* How the chunk-64 matrix-core prompt kernel spreads one (sequence, head)
 * over workgroups (see gdn_chunk_prefill_ex). */
typedef enum {
    GDN_COLUMNS_DEFAULT = 0,        /* the library's choice */
    GDN_COLUMNS_WHOLE = 1,          /* one workgroup per (sequence, head) */
    GDN_COLUMNS_SPLIT = 2           /* two workgroups of 64 value columns each */
} gdn_columns;

/* Library ABI version (increments on any signature change). */
int gdn_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char *gdn_status_string(int status);

/*
 * gdn_chunk_prefill -- run the recurrence over whole prompts with the
 * chunkwise-parallel form of the same page (G = cumsum g inside each chunk;
 * N = diag(beta)[exp(G_t - G_j) k_t.k_j]_{j<t}; D = (I+N)^-1 diag(beta)
 * (V - diag(exp G) K S0); O = diag(exp G) Q S0 + [exp(G_t - G_j) q_t.k_j]_{j<=t} D;
 * S_T = exp(G_last) S0 + K^T diag(exp(G_last - G)) D), which reaches the
 * per-token result above up to rounding.  The chunks of one sequence are walked
 * in order with the state kept on chip; the state touches device memory once
 * on entry and once on exit.  A sequence whose length is not a multiple of
 * `chunk` ends in a partial chunk whose missing rows act as the page's
 * token_valid padding (g = 0, beta = 0): they leave the state untouched and
 * produce no output rows.
 *
 *   q, k        [B, T, H, 128] io_dtype   (packed: [1, T, H, 128])
 *   v           [B, T, H, 128] io_dtype
 *   g, beta     [B, T, H] fp32
 *   S0          [N, H, 128, 128] fp32, or NULL for a zero initial state
 *   cu_seqlens  NULL: N = B sequences of T tokens each (B_or_N = B).
 *               Otherwise a device array of N+1 int32 offsets (B_or_N = N) into
 *               one packed batch of T tokens: sequence n owns tokens
 *               cu_seqlens[n] .. cu_seqlens[n+1]-1 and starts from S0[n].  The
 *               offsets must start at 0, never decrease and end at T; they are
 *               read on the device and clamped to [0, T], so a bad array gives
 *               wrong results, never an out-of-bounds access.  Zero-length
 *               sequences are allowed (S_T[n] = S0[n], no rows of O).  For
 *               debugging, with the environment variable GDN_CHECK_SEQLENS
 *               set (to anything but "0"), every call that takes cu_seqlens
 *               copies it to the host first, synchronising the stream (so not
 *               under graph capture), and returns GDN_ERR_INVALID_ARG, with
 *               nothing enqueued, for offsets that do not start at 0, decrease,
 *               or do not end at T.
 *   chunk       16, 32 or 64 (the page's prompt-block sizes); the result does
 *               not depend on it beyond rounding, so it is a tiling choice.  A
 *               bf16 batch of short sequences (at most 16 tokens per sequence
 *               on average: T <= 16 for a uniform batch, T <= 16 N for a packed
 *               one, as in a speculative verify pass) is tiled by 16 whatever
 *               the chunk, on a kernel that runs two sequence-heads per CU.
 *   O           same shape and dtype as v (fp32 with GDN_BF16_F32_OUT); rows of
 *               the call's tokens are all written.
 *   S_T         [N, H, 128, 128] fp32, the state after each sequence's last
 *               token.  S_T may be exactly S0 (in-place update of a prefix
 *               state); any other overlap of S_T with S0 is GDN_ERR_ALIAS.
 *               Keep them distinct to retain a snapshot of S0.
 *   O must not overlap q, k, v, g, beta, S0 or S_T; S_T must not overlap the
 *   token inputs (GDN_ERR_ALIAS).
 */
int gdn_chunk_prefill(const void *q, const void *k, const void *v, int io_dtype,
                      const float *g, const float *beta, const float *S0,
                      const int32_t *cu_seqlens, int64_t B_or_N, int64_t T,
                      int64_t H, int64_t dk, int64_t dv, int64_t chunk,
                      void *O, float *S_T, void *stream);

/*
 * gdn_chunk_prefill_ex -- gdn_chunk_prefill with a choice of how (I + N)^-1 is
 * formed.  The Qwen3.5-9B-npu model page ("How it works" -> "Gated DeltaNet on
 * the NPU") computes the triangular inverse by exact block doubling,
 * (D + C)^-1 = D^-1 - D^-1 C D^-1, from 1 x 1 blocks up; gdn_chunk_prefill by
 * default builds each 16 x 16 diagonal block that way on the matrix cores
 * (GDN_INVERSE_DOUBLING) and applies the block structure above it by block
 * forward substitution.  GDN_INVERSE_SUBSTITUTION forms the diagonal blocks by
 * fp32 back substitution instead.  Both reach the same result up to rounding.
 *
 * It also chooses how a (sequence, head) is spread over workgroups.  In that
 * statement of the chunk form every value column j of O, D and the state
 * depends only on column j of V and of S0, so the 128 columns can be walked
 * by separate workgroups that each repeat the key-side work (the Gram tiles,
 * the triangular inverse).  GDN_COLUMNS_SPLIT runs two workgroups of 64
 * columns per (sequence, head): each walks the chunks with half the
 * state-side work, which shortens the serial chain of a call that leaves CUs
 * idle (few sequences and heads) at the price of repeating the key-side work.
 * GDN_COLUMNS_DEFAULT splits exactly when the split launch still fits the
 * device's CUs at once (2 B_or_N H <= CUs); gdn_chunk_prefill takes that
 * default.
 *
 * Both choices apply to bf16 inputs at chunk 64 (the matrix-core kernel), and
 * naming either (anything but a DEFAULT) keeps such calls on that kernel even
 * for batches of short sequences; the other configurations substitute column
 * by column and ignore them.
 *
 *   inverse     a gdn_inverse value (else GDN_ERR_UNSUPPORTED).
 *   columns     a gdn_columns value (else GDN_ERR_UNSUPPORTED).
 *   Every other argument: as for gdn_chunk_prefill.
 */
int gdn_chunk_prefill_ex(const void *q, const void *k, const void *v, int io_dtype,
                         const float *g, const float *beta, const float *S0,
                         const int32_t *cu_seqlens, int64_t B_or_N, int64_t T, int64_t H,
                         int64_t dk, int64_t dv, int64_t chunk, int inverse, int columns,
                         void *O, float *S_T, void *stream);

/*
 * gdn_chunk_prefill_segmented -- gdn_chunk_prefill with each sequence cut into
 * segments of segment_len tokens that are walked in parallel.  Over a segment
 * the recurrence is affine in the entering state, S_out = M S_in + B (the
 * prompt form's state update, Qwen3.5-9B-npu model page, "How it works" ->
 * "Gated DeltaNet on the NPU", composed over the segment's chunks).  The call
 * runs the prompt form over all segments at once three times -- for B (from a
 * zero state), for M (with v = 0 from the identity) and, after a scan
 * S_in(p+1) = M_p S_in(p) + B_p over each sequence's segments, for O and the end
 * states from the true S_in -- so that a batch of a few long sequences keeps
 * every CU busy.  The result equals gdn_chunk_prefill's up to rounding (the scan
 * adds one fp32 product per segment boundary).  It triples the prompt-form
 * work, so it pays only when the plain call would leave most CUs idle.
 *
 *   q, k, v, g, beta, S0, cu_seqlens, B_or_N, T, H, dk, dv, chunk, O, S_T: as for
 *               gdn_chunk_prefill, uniform or packed.  Each sequence gets
 *               max(1, ceil(length / segment_len)) segments.
 *   segment_len a positive multiple of chunk.  A uniform batch with
 *               T <= segment_len is the plain gdn_chunk_prefill and needs no
 *               workspace.
 *   workspace   caller-owned device memory of at least
 *               gdn_chunk_prefill_segmented_workspace(io_dtype, cu_seqlens,
 *               B_or_N, T, H, segment_len) bytes, 256-byte aligned, overlapping
 *               no argument; its contents are scratch between calls.  Calls
 *               sharing a workspace must not run concurrently.
 *   workspace_bytes  its size.
 *   The token rows (B * T, or T when packed) must be below 2^31: the segments'
 *   offsets are int32.
 *   GDN_ERR_INVALID_ARG for a bad segment_len, too many rows, or a missing or
 *   short workspace; GDN_ERR_ALIAS if the workspace overlaps an argument.
 */
int gdn_chunk_prefill_segmented(const void *q, const void *k, const void *v, int io_dtype,
                                const float *g, const float *beta, const float *S0,
                                const int32_t *cu_seqlens, int64_t B_or_N, int64_t T, int64_t H,
                                int64_t dk, int64_t dv, int64_t chunk, int64_t segment_len,
                                void *workspace, int64_t workspace_bytes, void *O, float *S_T,
                                void *stream);

/*
 * gdn_chunk_prefill_segmented_noalloc -- gdn_chunk_prefill_segmented without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that must not allocate, harnesses
 * that forbid it).  The scratch is a file-scope device array in libgdn,
 * gdn_noalloc_scratch_bytes() bytes (48 MiB + 64 KiB), one copy per GPU,
 * held while the library is loaded; its address is looked up once per device
 * on that device's first call.  The call allocates nothing.
 *
 *   Arguments, layouts and results as gdn_chunk_prefill_segmented.  A call
 *   whose workspace (gdn_chunk_prefill_segmented_workspace) would exceed the
 *   scratch returns GDN_ERR_SCRATCH with nothing enqueued; that is about
 *   256 (segment, head) pairs, e.g. 16 heads of a 4096-token sequence in
 *   256-token segments.
 *   Every call on one GPU uses the same scratch: calls that overlap in time
 *   on one GPU (on different streams, or from different host threads without
 *   ordering) race and give wrong results.  Calls in one stream are ordered
 *   and safe.  Nothing in the scratch needs to start at zero (each call
 *   writes every part it reads).
 */
int gdn_chunk_prefill_segmented_noalloc(const void *q, const void *k, const void *v, int io_dtype,
                                        const float *g, const float *beta, const float *S0,
                                        const int32_t *cu_seqlens, int64_t B_or_N, int64_t T,
                                        int64_t H, int64_t dk, int64_t dv, int64_t chunk,
                                        int64_t segment_len, void *O, float *S_T, void *stream);

/* Bytes of device scratch gdn_chunk_prefill_segmented_noalloc holds per GPU. */
int64_t gdn_noalloc_scratch_bytes(void);

/* Bytes of workspace gdn_chunk_prefill_segmented needs for these sizes, or -1
 * if they are invalid: per segment and head, three states of 64 KiB (a
 * uniform batch has B ceil(T / segment_len) segments; a packed one is sized
 * for N + ceil(T / segment_len)), plus a zero copy of v and the segments'
 * offsets.  cu_seqlens is not read: only whether it is NULL matters. */
int64_t gdn_chunk_prefill_segmented_workspace(int io_dtype, const int32_t *cu_seqlens,
                                              int64_t B_or_N, int64_t T, int64_t H,
                                              int64_t segment_len);

/*
 * gdn_chunk_prefill_gated -- gdn_chunk_prefill with the gated RMS norm that
 * follows the recurrence in a Gated DeltaNet block (Qwen3.5-4B -- Hexagon NPU
 * (QHexRT) -- v81 page, the opening description of the text decoder: a short
 * convolution window carried between calls, the recurrent state and a gated
 * RMS norm) applied to each output row before it is rounded and stored:
 *
 *     y = norm_w * o / sqrt(mean(o^2) + eps) * silu(z),  silu(x) = x / (1 + exp(-x))
 *
 * with the mean over the 128 values of one token row of one head.  The norm is
 * scale-invariant up to eps (the Qwen3.5-9B-npu model page, "How it works" ->
 * "fp16 precision of the DeltaNet output", scales q by 1024 and eps by 1024^2
 * for exactly that reason), so it takes the fp32 O before any rounding.
 *
 *   q, k, v, g, beta, S0, cu_seqlens, B_or_N, T, H, dk, dv, chunk, S_T: as for
 *               gdn_chunk_prefill.
 *   z           [B, T, H, 128] io_dtype, 16-byte aligned; NULL only when the call
 *               has no token rows.
 *   norm_w      [128] fp32, one weight vector shared by all heads, 4-byte aligned.
 *   eps         finite and >= 0 (else GDN_ERR_INVALID_ARG); with eps = 0 an
 *               all-zero output row gives NaN.
 *   Y           same shape and dtype as v: the normed rows (O itself is not
 *               written anywhere).
 *   Y must not overlap any input, z, norm_w or S_T; S_T must not overlap z or
 *   norm_w (GDN_ERR_ALIAS), besides the rules of gdn_chunk_prefill.
 */
int gdn_chunk_prefill_gated(const void *q, const void *k, const void *v, int io_dtype,
                            const float *g, const float *beta, const float *S0,
                            const int32_t *cu_seqlens, int64_t B_or_N, int64_t T,
                            int64_t H, int64_t dk, int64_t dv, int64_t chunk,
                            const void *z, const float *norm_w, float eps, void *Y,
                            float *S_T, void *stream);

/*
 * gdn_prefill_states -- the prompt form that also keeps the state after every
 * token.  The Qwen3.5-9B-npu model page (section "New in v2", the prompt
 * lookup decoding item) checks a block of drafted tokens in one pass and,
 * since a DeltaNet state cannot be rewound, snapshots the state first and
 * re-feeds the accepted tokens.  With the state after each token kept,
 * the caller takes S_tok at the last accepted token instead: no snapshot and no
 * second pass.  Each token applies the page's one-token matrix form (as
 * gdn_decode_step) to a state kept on chip; the result equals gdn_chunk_prefill's
 * up to rounding.
 *
 *   q, k, v, g, beta, S0, cu_seqlens, B_or_N, T, H, dk, dv, O: as for
 *               gdn_chunk_prefill (there is no chunk argument).
 *   S_tok       [B, T, H, 128, 128] fp32 (packed: [1, T, H, 128, 128]): for each
 *               token row and head, the state after that token within its
 *               sequence (so a sequence's last row holds its final state).
 *               64 KiB per token and head is written.
 *   O and S_tok must not overlap each other, the inputs or S0 (GDN_ERR_ALIAS).
 */
int gdn_prefill_states(const void *q, const void *k, const void *v, int io_dtype,
                       const float *g, const float *beta, const float *S0,
                       const int32_t *cu_seqlens, int64_t B_or_N, int64_t T,
                       int64_t H, int64_t dk, int64_t dv, void *O, float *S_tok,
                       void *stream);

/*
 * gdn_preop -- the block's pre-operations, from the per-token projections to the
 * recurrence's inputs, in one pass.  The Qwen3.5-4B -- Hexagon NPU (QHexRT) --
 * v81 page lists a causal convolution over a short window carried between calls,
 * the recurrent state and a gated RMS norm; the QCS6490 page's port notes name
 * Softplus among the gate's operations.  For
 * each stream x of q, k, v and channel c, with rows before a sequence's first
 * token taken from its FIFO state:
 *
 *     conv_t[c] = sum_{j=0..3} conv_w[c][j] x_{t-3+j}[c],   y_t = silu(conv_t)
 *     q_t, k_t  = y_t / sqrt(sum_c y_t[c]^2 + eps),          v_t = y_t
 *     g_t = -softplus(a_t),   beta_t = sigmoid(b_t)
 *
 * and the FIFO afterwards holds each sequence's last three raw rows (the
 * newest rows of [state_in; the sequence's rows]).  The outputs are exactly
 * gdn_chunk_prefill's (or, with one token per sequence, gdn_decode_step's)
 * inputs.
 *
 *   xq, xk, xv  [B, T, H, 128] io_dtype (packed: [1, T, H, 128]), 16-byte aligned
 *   a, b        [B, T, H] fp32
 *   conv_w      [3, H, 128, 4] fp32 (streams q, k, v; taps oldest first), 16-byte aligned
 *   state_in    [N, 3, H, 3, 128] io_dtype, rows oldest first; state_out the same
 *               shape, either exactly state_in (updated in place) or disjoint
 *   cu_seqlens, B_or_N, T, H: as for gdn_chunk_prefill; dk = dv = 128 and
 *               kernel_size = 4 (else GDN_ERR_UNSUPPORTED)
 *   eps         finite and >= 0
 *   q, k, v     like xq; g, beta like a
 *   No output may overlap an input or another output, save state_out == state_in
 *   (GDN_ERR_ALIAS).
 */
int gdn_preop(const void *xq, const void *xk, const void *xv, int io_dtype, const float *a,
              const float *b, const float *conv_w, const void *state_in, void *state_out,
              const int32_t *cu_seqlens, int64_t B_or_N, int64_t T, int64_t H, int64_t dk,
              int64_t dv, int64_t kernel_size, float eps, void *q, void *k, void *v, float *g,
              float *beta, void *stream);

/*
 * gdn_chunk_prefill_preop -- gdn_preop and gdn_chunk_prefill (chunk 64) as one
 * prompt-form call from the raw projections: the pre-operations (gdn_preop's
 * formulas and page citations: the causal conv over the FIFO window, silu,
 * q and k divided by sqrt(sum y^2 + eps), g = -softplus(a), beta = sigmoid(b))
 * run inside the 64-token matrix-core kernel as it loads each chunk, so q, k,
 * v, g and beta never go to memory.  q and k enter the recurrence's products
 * rounded from fp32 to fp16, v rounded to bf16 (the prompt form's own operand
 * types), instead of all three rounded to bf16 in between as with two calls.
 * The FIFO state is then advanced as by gdn_preop.
 *
 *   xq, xk, xv, a, b, conv_w, state_in, state_out, eps, kernel_size: as for
 *               gdn_preop, with io_dtype GDN_BF16 only
 *   S0, cu_seqlens, B_or_N, T, H, dk, dv, O, S_T: as for gdn_chunk_prefill
 *               (O bf16), with chunk 64 only
 *   Other io dtypes, chunks or kernel sizes: GDN_ERR_UNSUPPORTED.  O and S_T
 *   must not overlap the inputs (gdn_chunk_prefill's rule, conv_w and state_in
 *   included); state_out is exactly state_in (advanced in place) or overlaps
 *   nothing (GDN_ERR_ALIAS).
 */
int gdn_chunk_prefill_preop(const void *xq, const void *xk, const void *xv, int io_dtype,
                            const float *a, const float *b, const float *conv_w,
                            const void *state_in, void *state_out, float eps, const float *S0,
                            const int32_t *cu_seqlens, int64_t B_or_N, int64_t T, int64_t H,
                            int64_t dk, int64_t dv, int64_t kernel_size, int64_t chunk, void *O,
                            float *S_T, void *stream);

/*
 * gdn_decode_step -- one token per (sequence, head) with the page's one-token
 * matrix form: with d = exp(g), a = S^T k and b = S^T q read in one pass over
 * S, delta = beta (v - d a), o = d b + (q.k) delta and S' = d S + k delta^T,
 * written back in place.  Each state is read once and written once.
 *
 *   q, k     [B, H, 128] io_dtype      v  [B, H, 128] io_dtype
 *   g, beta  [B, H] fp32
 *   S        [B, H, 128, 128] fp32, read and overwritten in place
 *   o        [B, H, 128] io_dtype
 *   o must not overlap S or the inputs, and S must not overlap the inputs
 *   (GDN_ERR_ALIAS).
 */
int gdn_decode_step(const void *q, const void *k, const void *v, int io_dtype,
                    const float *g, const float *beta, float *S, int64_t B,
                    int64_t H, int64_t dk, int64_t dv, void *o, void *stream);

/* How gdn_decode_step_ex moves the state. */
typedef enum {
    GDN_STATE_CACHED = 0,      /* plain loads and stores (gdn_decode_step) */
    GDN_STATE_STREAMING = 1    /* non-temporal loads and stores */
} gdn_state_hint;

/*
 * gdn_decode_step_ex -- gdn_decode_step with a choice of how the state is
 * loaded and stored; the arithmetic, and so the result, is the same bit for bit.
 * A model steps many layers' states in turn, so by the time a layer's state is
 * read again it has left the last-level cache; for that case
 * GDN_STATE_STREAMING moves it with non-temporal loads and stores (and one
 * workgroup per head state), which on MI355X streams it faster (64 x 16 heads:
 * 24.0 against 29.0 us per step when eight such batches take turns).  When one
 * batch small enough for the cache is stepped over and over, GDN_STATE_CACHED
 * is faster (22.6 against 23.0 us).
 *
 *   state_hint  a gdn_state_hint value (else GDN_ERR_UNSUPPORTED).
 *   Every other argument: as for gdn_decode_step.
 */
int gdn_decode_step_ex(const void *q, const void *k, const void *v, int io_dtype,
                       const float *g, const float *beta, float *S, int64_t B,
                       int64_t H, int64_t dk, int64_t dv, int state_hint, void *o,
                       void *stream);

/*
 * gdn_decode_step_preop -- the decode step with the block's pre-operations
 * fused in front: from the raw per-token projections and gate inputs of one
 * token per (sequence, head), with each sequence's conv FIFO read and advanced,
 * to o and the updated state, in one launch.  The pre-operations are
 * gdn_preop's (its page citations and formulas): a causal conv over the three
 * FIFO rows and the token, silu, q and k divided by sqrt(sum y^2 + eps),
 * g = -softplus(a), beta = sigmoid(b); the step is gdn_decode_step's.  q, k and
 * v are kept in fp32 between the two, so the result is gdn_preop followed by
 * gdn_decode_step without the rounding of q, k, v to the io dtype in between.
 *
 *   xq, xk, xv  [B, H, 128] io_dtype, 16-byte aligned
 *   a, b        [B, H] fp32
 *   conv_w      [3, H, 128, 4] fp32, 16-byte aligned (as for gdn_preop)
 *   state_in    [B, 3, H, 3, 128] io_dtype, rows oldest first; state_out the
 *               same shape, either exactly state_in (advanced in place) or
 *               disjoint
 *   eps         finite and >= 0
 *   z, norm_w, norm_eps  NULL z gives the step's o.  Otherwise o receives the
 *               block's gated RMS norm of it, as gdn_chunk_prefill_gated
 *               applies it: y = norm_w o / sqrt(mean(o^2) + norm_eps) silu(z),
 *               on the fp32 o, with z [B, H, 128] io_dtype (16-byte aligned),
 *               norm_w [128] fp32 and norm_eps finite and >= 0.
 *   S, B, H, dk, dv, o: as for gdn_decode_step; state_hint as for
 *               gdn_decode_step_ex.
 *   o, S and state_out must not overlap the inputs (z and norm_w included) or
 *   each other (save state_out == state_in) (GDN_ERR_ALIAS).
 */
int gdn_decode_step_preop(const void *xq, const void *xk, const void *xv, int io_dtype,
                          const float *a, const float *b, const float *conv_w,
                          const void *state_in, void *state_out, float eps, const void *z,
                          const float *norm_w, float norm_eps, float *S, int64_t B, int64_t H,
                          int64_t dk, int64_t dv, int state_hint, void *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
