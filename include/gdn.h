/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta rule forward library.
 *
 * The operation is the chunked gated delta rule of the MaxText PR "Add
 * context parallelism to the Gated Delta Net (Qwen3-Next / Qwen3.5)":
 *   - per chunk of C tokens, the WY factors w, u of the affine chunk map
 *     h_out = (gamma I - k_tilde^T w) h + k_tilde^T u = M h + U and the chunk
 *     output o = (q_g - attn_i w) h + attn_i u (section "Why");
 *   - the sequential scan of that map over chunks;
 *   - the three-phase segment pass (section "Implementation"): a zero-state
 *     pass carrying M (low-rank update M <- gamma M - k_tilde^T (w M)), an
 *     exclusive prefix scan over the (M_r, U_r) pairs, and a re-pass from the
 *     true incoming state;
 *   - the single-token recurrent decode step on the fp32 state, whose layout
 *     [H_v, K, V] f32 per request follows "RFC(qwen35): TP Phase 2",
 *     section "Partition Contract".
 *
 * Per token (K-major state h in R^{K x V}):
 *   h <- exp(g_t) h;  delta = beta_t (v_t - h^T k_t);  h <- h + k_t delta^T;
 *   o_t = h^T q_t.
 * The query is used unscaled: a caller wanting 1/sqrt(K) pre-scales q.
 *
 * Conventions for every entry point
 *   - Tensors are caller-owned device buffers, row-major, contiguous, 16-byte
 *     aligned.  The library allocates nothing and keeps no state apart from a
 *     thread-local error message.
 *   - q, k, v and o share one dtype (GDN_F32 or GDN_BF16).  g (log-decay,
 *     alpha = exp(g)) and beta are fp32.  Every state, M and U is fp32.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work
 *     and return without synchronising.
 *   - Every argument is checked before anything is launched; a call that
 *     returns an error has written nothing.  HIP launch failures surface as
 *     GDN_ELAUNCH.  No C++ exception crosses the ABI.
 *   - Supported (K, V, C): (32, 32, 16) and (128, 128, 64).  Anything else is
 *     GDN_EUNSUPPORTED; there is no fallback.
 *   - The kernels address one chunk of C token rows with 32-bit offsets, so a
 *     problem whose C rows of q, k (H_qk heads) or of v, o (H heads) span
 *     2 GiB or more is GDN_EUNSUPPORTED (H of 131072 or more at K = V = 128,
 *     C = 64 in bf16).
 *   - The decay g may have either sign and beta any value on every path; the
 *     method's own ranges are g <= 0 (alpha = exp(g) in (0, 1]) and
 *     0 <= beta <= 1.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_EINVAL = 1,        /* null pointer, bad size, misaligned buffer          */
    GDN_EUNSUPPORTED = 2,  /* shape / dtype combination not built                */
    GDN_EORDER = 3,        /* segments or sequence offsets not contiguous+ordered */
    GDN_ELAUNCH = 4,       /* HIP reported an error at launch                    */
    GDN_EWORKSPACE = 5     /* a workspace buffer is smaller than the problem needs */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum gdn_scan_mode {
    GDN_SCAN_EMIT = 0,   /* outputs o and the final state                           */
    GDN_SCAN_CARRY = 1,  /* zero-state pass per segment emitting (M_r, U_r), no o   */
    GDN_SCAN_HEAD_EMIT_CARRY = 2, /* segment 0 emitted, segments 1 .. R-1 carried */
    GDN_SCAN_TAIL_EMIT = 3        /* packed pieces: every piece but the first emitted */
} gdn_scan_mode;

#define GDN_MAX_SEQS 256
#define GDN_MAX_SEGMENTS 64

/*
 * Problem description (host memory; read during the call only).
 *
 * Batch mode (n_seqs == 0): B independent sequences of S tokens each;
 *   q, k [B,S,H,K]; v, o [B,S,H,V]; g, beta [B,S,H]; states [B,H,K,V].
 * Packed mode (n_seqs > 0, B == 1): n_seqs sequences laid end to end on one
 *   token axis of S tokens, sequence n owning tokens cu_seqlens[n] ..
 *   cu_seqlens[n+1]-1 (cu_seqlens[0] == 0, non-decreasing, cu_seqlens[n_seqs]
 *   == S, at most GDN_MAX_SEQS sequences); q, k [S,H,K], ...; states
 *   [n_seqs,H,K,V].  Sequences need not be multiples of C: a ragged tail is
 *   masked exactly like padding (g = 0, q = k = v = 0, beta = 0), which the
 *   MaxText PR ("Implementation") shows is a no-op for the recurrence.
 *
 * Grouped heads: q and k may have H_qk heads for the H value heads (v, o,
 *   g, beta and every state have H), H a multiple of H_qk; value head h reads
 *   key head h / (H / H_qk), each key head serving H / H_qk consecutive value
 *   heads (the separate key and value head counts of "RFC(qwen35): TP Phase
 *   2", section "Partition Contract"; the grouped order of the Ulysses
 *   context-parallelism page).  q, k are then [B,S,H_qk,K] ([S,H_qk,K]
 *   packed).  H_qk == 0 means H_qk = H.  Anything else is GDN_EINVAL.
 *
 * Segments (batch mode only): every sequence is cut into n_segments
 *   contiguous, in-order pieces starting at seg_starts[r] (relative to the
 *   sequence start).  seg_starts[0] == 0, strictly increasing, multiples of
 *   C, all < S, otherwise GDN_EORDER -- a sequential recurrence needs
 *   contiguous, in-order slices (MaxText PR, section "Limitation").
 *   seg_starts == NULL splits the chunks as evenly as possible.
 *   Packed mode requires n_segments == 1.
 *
 * Pieces (packed mode only): the segments of a packed batch, sized per
 *   sequence so that one long sequence does not set the time of the whole
 *   batch (its chunks are sequential; the segment pass of the MaxText PR,
 *   section "Implementation", turns them into parallel chains).  With
 *   max_piece_chunks = m > 0, a sequence of c > m chunks is cut into
 *   R_n = ceil(c / m) pieces, piece s starting at chunk floor(s * c / R_n) of
 *   the sequence; every other sequence is one piece.  m == 0 makes every
 *   sequence one piece.  Pieces are numbered in token order; their count P
 *   (gdn_num_pieces) must not exceed GDN_MAX_SEQS.  Per-piece buffers are
 *   [P,H,...]; sequence n's pieces are consecutive.  Batch mode requires
 *   max_piece_chunks == 0.
 */
typedef struct gdn_problem {
    int32_t B, S, H, K, V, C;
    int32_t dtype;                /* gdn_dtype of q, k, v, o and of the WY workspace */
    int32_t n_seqs;               /* 0: batch mode; >0: packed mode                 */
    const int32_t *cu_seqlens;    /* host pointer, n_seqs + 1 entries (packed mode) */
    int32_t n_segments;           /* R >= 1                                          */
    const int32_t *seg_starts;    /* host pointer, R entries, or NULL                */
    int32_t max_piece_chunks;     /* packed mode: longest piece in chunks, 0 = none  */
    int32_t H_qk;                 /* heads of q and k; 0 = H (see grouped heads)     */
} gdn_problem;

/* Check a problem description without touching the GPU. */
gdn_status gdn_validate(const gdn_problem *p);

/* Number of pieces P of a packed problem (n_seqs when max_piece_chunks == 0);
 * the number of segments B * R of a batch problem; -1 if p is invalid. */
int32_t gdn_num_pieces(const gdn_problem *p);

/* Bytes of the WY workspace written by gdn_chunk_prepare: for every chunk
 * (batch: B * ceil(S/C); packed: sum over sequences of ceil(len/C)) and head,
 * w [C,K] then, after all w blocks, u [C,V], in the problem's dtype.
 * Returns 0 for an invalid problem. */
size_t gdn_wy_workspace_bytes(const gdn_problem *p);

/* Bytes of the segment transition pairs M [R,N,H,K,K] plus U [R,N,H,K,V]
 * (fp32; N = B or n_seqs): R*N*H*K*(K+V)*4, independent of S -- the
 * sequence-length-independent cross-rank payload of the MaxText PR
 * ("Measured results", "Tests").  Packed problems: P*H*K*(K+V)*4 for the P
 * pieces.  Returns 0 for an invalid problem. */
size_t gdn_segment_workspace_bytes(const gdn_problem *p);

/*
 * gdn_chunk_prepare -- per-chunk WY factors (MaxText PR, "Why": the w and u
 * of the affine chunk form; "Implementation": _gdn_chunk_prepare).
 * For each chunk and head, with G the within-chunk cumulative log-decay:
 *   A[r,s] = beta_r exp(G_r - G_s) k_r.k_s (s < r),  T = (I + A)^{-1},
 *   w = T diag(beta exp(G)) K_c,  u = T diag(beta) V_c.
 * k, v, g, beta as in the problem; wy receives gdn_wy_workspace_bytes(p)
 * bytes (w blocks [n_chunks,H,C,K] followed by u blocks [n_chunks,H,C,V]).
 * wy_bytes is the size of the buffer at wy: GDN_EWORKSPACE (nothing written)
 * when it is smaller than gdn_wy_workspace_bytes(p).
 * Rows past the end of a ragged chunk are zero.  Segments are ignored.
 */
gdn_status gdn_chunk_prepare(const gdn_problem *p, const void *k, const void *v,
                             const float *g, const float *beta, void *wy, size_t wy_bytes,
                             void *stream);

/*
 * gdn_scan -- the inter-chunk affine scan (MaxText PR, "Why" equations;
 * "Implementation" phases 1 and 3).
 *
 * wy: NULL recomputes the WY factors inside the scan; otherwise a workspace
 *   filled by gdn_chunk_prepare for the same problem and inputs is reused.
 *   wy_bytes is the size of the buffer at wy (ignored when wy is NULL):
 *   GDN_EWORKSPACE when it is smaller than gdn_wy_workspace_bytes(p).
 *
 * GDN_SCAN_EMIT: for every segment r of every sequence n, starts from
 *   h_in[r,n] (h_in [R,N,H,K,V] fp32; NULL = zero state for every segment),
 *   runs the chunk map over the segment, writes o for its tokens, and the
 *   last segment writes the final state to h_out [N,H,K,V] (nullable).
 *   h_out may alias h_in only when R == 1.  q, o required.
 * GDN_SCAN_CARRY: for every segment, a zero-state pass carrying the composed
 *   transition: writes M_out [R,N,H,K,K] and U_out [R,N,H,K,V] with
 *   h_end = M_r h_start + U_r.  q, o, h_in, h_out are ignored.
 * GDN_SCAN_HEAD_EMIT_CARRY (batch mode, R >= 2): phase 1 of the segment pass
 *   without its redundant piece.  Segment 0's incoming state is known, so it
 *   is emitted as in GDN_SCAN_EMIT from h_in [N,H,K,V] (NULL = zero): o for its
 *   tokens (the rest of o is not written) and its final state, the state
 *   entering segment 1, to h_out [N,H,K,V] (nullable).  Segments 1 .. R-1 are
 *   carried as in GDN_SCAN_CARRY into M_out [R-1,N,H,K,K] and
 *   U_out [R-1,N,H,K,V] (slot r-1 for segment r).  On the matrix-core path
 *   (bf16, K = V = 128, C = 64) this is one launch.  GDN_EINVAL for batch
 *   problems with R < 2.
 *
 * Packed problems work on pieces (P of them, see gdn_problem):
 *   GDN_SCAN_EMIT and GDN_SCAN_CARRY run every piece, with h_in, M_out and
 *   U_out indexed by piece ([P,H,...]); the last piece of sequence n writes
 *   h_out[n] ([N,H,K,V]).
 *   GDN_SCAN_HEAD_EMIT_CARRY emits the first piece of every sequence from
 *   h_in[n] ([N,H,K,V], NULL = zero) and writes the state at its end to
 *   h_out[n] (the final state when the sequence is one piece), and carries
 *   pieces 1 .. R_n-2 of every sequence into M_out, U_out [P,H,...] (slot =
 *   piece); the last piece of a sequence of R_n >= 2 pieces is not run.
 *   GDN_SCAN_TAIL_EMIT emits pieces 1 .. R_n-1 of every sequence from
 *   h_in [P,H,K,V] (slot = piece; the first pieces' slots are not read) and
 *   writes each such sequence's final state to h_out[n]; one-piece sequences
 *   are not touched.  GDN_EINVAL for batch problems (slice the tensors
 *   instead).
 *   Together: HEAD_EMIT_CARRY, gdn_piece_compose(first = 1), TAIL_EMIT is the
 *   segment pass without redundant work; CARRY, gdn_piece_compose(first = 0),
 *   EMIT is the plain one.
 *   Work items are ordered longest first, so long pieces start first.
 */
gdn_status gdn_scan(const gdn_problem *p, int32_t mode,
                    const void *q, const void *k, const void *v,
                    const float *g, const float *beta, const void *wy, size_t wy_bytes,
                    const float *h_in, void *o, float *h_out,
                    float *M_out, float *U_out, void *stream);

/*
 * gdn_forward -- the whole chunked forward of a problem in one call: outputs
 * o and final states h_out from inputs q, k, v, g, beta and initial states h0
 * (nullable = zero), with the WY factors recomputed inside the scans.
 *   - One chain per sequence (batch with n_segments == 1, or packed with no
 *     sequence cut into pieces): the emitting scan alone (gdn_scan
 *     GDN_SCAN_EMIT).
 *   - Segments (batch, R >= 2): the three-phase pass of the MaxText PR,
 *     section "Implementation", without its redundant work: segment 0 emitted
 *     from h0 beside the carrying pass of segments 1 .. R-2, the exclusive
 *     prefix scan of their (M_r, U_r) seeded with segment 0's final state, and
 *     the emitting pass of segments 1 .. R-1 (GDN_SCAN_HEAD_EMIT_CARRY,
 *     gdn_segment_compose, GDN_SCAN_EMIT).
 *   - Packed pieces (max_piece_chunks): GDN_SCAN_HEAD_EMIT_CARRY,
 *     gdn_piece_compose(first = 1), GDN_SCAN_TAIL_EMIT.
 * Layouts as gdn_scan; h0, h_out [N,H,K,V] fp32, h_out nullable and allowed to
 * alias h0 (in-place continuation).  workspace: caller-owned device memory of
 * gdn_forward_workspace_bytes(p) bytes, 16-byte aligned, not overlapping o,
 * h0 or h_out (contents undefined on return; NULL allowed when that size is
 * 0); GDN_EWORKSPACE when workspace_bytes is smaller.  The workspace holds the
 * (M, U) pairs and the incoming states of the segments or pieces, whose size
 * does not depend on S.  Errors as gdn_scan; nothing is written on failure.
 */
size_t gdn_forward_workspace_bytes(const gdn_problem *p);
gdn_status gdn_forward(const gdn_problem *p, const void *q, const void *k, const void *v,
                       const float *g, const float *beta, const float *h0, void *o, float *h_out,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_forward_noalloc -- gdn_forward without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace is a
 * file-scope device array of GDN_FORWARD_SCRATCH_BYTES (64 MiB) inside the
 * library, one per GPU it runs on (on the device of `stream`), held until the
 * process ends; the call allocates nothing.  A problem whose
 * gdn_forward_workspace_bytes exceeds it is GDN_EWORKSPACE (the 64k-token,
 * 32-head, K = V = 128 forward in 4 segments needs 16 MiB; R segments of N
 * sequences need about (3R - 4) * N * H * K * V * 4 bytes).  Every call on a
 * GPU uses the same array, so calls that overlap on one GPU (other streams or
 * threads) race: serialise them.  Otherwise as gdn_forward.
 */
#define GDN_FORWARD_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_forward_noalloc(const gdn_problem *p, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const float *h0, void *o, float *h_out,
                               void *stream);

/*
 * gdn_segment_compose -- exclusive prefix scan over segment pairs (MaxText
 * PR, "Implementation" phase 2):
 *   h_in[0] = h0 (NULL = zero), h_in[r+1] = M[r] h_in[r] + U[r],
 *   h_final = M[R-1] h_in[R-1] + U[R-1] (nullable output).
 * M [R,N,H,K,K], U and h_in [R,N,H,K,V], h0 and h_final [N,H,K,V], fp32.
 * h_in must not alias M, U or h0.
 */
gdn_status gdn_segment_compose(int32_t R, int32_t N, int32_t H, int32_t K, int32_t V,
                               const float *M, const float *U, const float *h0,
                               float *h_in, float *h_final, void *stream);

/*
 * gdn_piece_compose -- the prefix scan of gdn_segment_compose run per
 * sequence of a packed problem over its pieces (pieces f_n .. f_n+R_n-1 of
 * sequence n, see gdn_problem), starting at piece `first` (0 or 1) of each:
 *   x = h_seed[n] (NULL = zero);  for s = first .. R_n-1:
 *     h_in[f_n+s] = x;  x = M[f_n+s] x + U[f_n+s] (skipped for s = R_n-1
 *     unless h_final);
 *   h_final[n] = x (nullable; h_seed[n] when first >= R_n).
 * first = 0 seeds every sequence with its initial state (after
 * GDN_SCAN_CARRY); first = 1 seeds it with the state after its first piece
 * (h_out of GDN_SCAN_HEAD_EMIT_CARRY), reading M, U of pieces 1 .. R_n-2 only.
 * M [P,H,K,K], U and h_in [P,H,K,V], h_seed and h_final [N,H,K,V], fp32.
 * h_in and h_final must not alias the inputs or each other.  GDN_EINVAL for
 * batch problems (use gdn_segment_compose).
 */
gdn_status gdn_piece_compose(const gdn_problem *p, int32_t first, const float *M, const float *U,
                             const float *h_seed, float *h_in, float *h_final, void *stream);

/*
 * gdn_decode_step -- one token per sequence, in place on the fp32 state
 * (the per-token recurrence above; the "GDR decode kernel" of
 * "RFC(qwen35): TP Phase 2", section "Kernel Work", state [H_v,K,V] f32).
 * q, k [B,H_qk,K]; v, o [B,H,V] in `dtype`; g, beta [B,H] fp32;
 * state [B,H,K,V] fp32, read and written once.  H_qk divides H (grouped heads
 * as in gdn_problem; pass H_qk = H for one key head per value head).
 */
gdn_status gdn_decode_step(int32_t B, int32_t H, int32_t H_qk, int32_t K, int32_t V, int32_t dtype,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta, float *state, void *o,
                           void *stream);

/*
 * gdn_causal_conv1d -- the depthwise causal convolution over the q, k, v
 * channels before the core (MaxText PR, section "Implementation": a causal
 * conv1d whose shard halo is W-1 tokens; "RFC(qwen35): TP Phase 2", section
 * "Partition Contract": a conv state of qkv_dim x (W-1) per request):
 *   y[t,c] = act( sum_{i<W} weight[c,i] * x~[t-(W-1)+i, c] ),
 * x~ being the sequence's tokens preceded by its state (the W-1 previous
 * tokens, oldest first; zeros when state_in is NULL); act is the identity
 * (activation 0) or SiLU(u) = u / (1 + e^-u) (activation 1).  state_out
 * (nullable) receives the last W-1 positions of x~, so a sequence can be
 * continued token by token (decode) or chunk by chunk.
 * Batch (cu_seqlens NULL): B sequences of S tokens, x, y [B,S,D].  Packed:
 * B == 1, n_seqs sequences at offsets cu_seqlens (host, n_seqs + 1 entries,
 * first 0, non-decreasing, last S), x, y [S,D].  weight [D,W]; states
 * [N,D,W-1] (N = B or n_seqs); all in `dtype`, accumulation in fp32.
 * 1 <= W <= 8.  y must not overlap x.  state_out may alias state_in only when
 * every sequence has at most 8 tokens and none crosses a multiple of 64 on the
 * token axis (one-token decode batches always qualify); otherwise GDN_EINVAL.
 */
gdn_status gdn_causal_conv1d(int32_t B, int32_t S, int32_t D, int32_t W, int32_t dtype, int32_t activation,
                             const int32_t *cu_seqlens, int32_t n_seqs, const void *x, const void *weight,
                             const void *state_in, void *state_out, void *y, void *stream);

/*
 * gdn_gated_rmsnorm -- the gated RMSNorm after the core ("RFC(qwen35): TP
 * Phase 2", section "Execution Contract"), per row of V elements:
 *   y = o / sqrt(mean(o^2) + eps) * weight * SiLU(z).
 * o, z, y [rows, V] in `dtype` (z nullable: no gate), weight [V] fp32,
 * 1 <= V <= 256, eps >= 0; accumulation in fp32.  y may alias o.
 */
gdn_status gdn_gated_rmsnorm(int64_t rows, int32_t V, int32_t dtype, float eps, const void *o, const void *z,
                             const float *weight, void *y, void *stream);

/*
 * gdn_backward -- gradients of a loss l(o, hT) through the forward of the
 * problem (batch or packed, grouped key heads included), given
 * dout = dl/do [same layout as o, `dtype`] and dhT = dl/dhT
 * ([N,H,K,V] fp32, nullable = zero).  Segments (batch) and pieces (packed)
 * schedule the two state scans as they do the forward's: every part of a
 * sequence is scanned at once, from boundary states composed of the parts'
 * affine carries (the state scan's M, U; the reverse scan's M^T and offset),
 * so a sequence of few heads still fills the GPU.  The result is that of one
 * chain per sequence up to fp32 rounding.  The MaxText PR "Add context
 * parallelism to the Gated Delta Net" tests a backward pass against the
 * single-device recurrence (section "Tests") without printing one; this is
 * the chain rule through the chunk equations of its section "Why".
 * With grouped key heads dq, dk of a key head are the sums over the value
 * heads that read it.
 * Outputs, each in the layout of its input: dq, dk, dv in `dtype`; dg,
 * dbeta fp32; dh0 [N,H,K,V] fp32 (nullable: not written; written whether or
 * not h0 is given).  h0 nullable (zero state).  Every output is fully
 * written for the real tokens; none may overlap an input.  workspace: caller
 * owned device memory of gdn_backward_workspace_bytes(p) bytes, 16-byte
 * aligned (contents undefined on return; it grows by P*H*(2*K*K + 4*K*V)*4
 * bytes when the P chains split the sequences).  Arithmetic is fp32
 * throughout, except that for bf16 inputs at K = V = 128 the Grams K K^T and
 * Q K^T multiply the bf16 values on the bf16 matrix cores (exact products,
 * fp32 sums), and the gradient products over the value axis take their fp32
 * operands as bf16 pairs hi + lo (within 2^-18 of the operand; products of
 * pairs are exact, sums fp32).
 * Errors as gdn_scan; nothing is written on failure.
 */
size_t gdn_backward_workspace_bytes(const gdn_problem *p);
gdn_status gdn_backward(const gdn_problem *p, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, const float *h0, const void *dout,
                        const float *dhT, void *dq, void *dk, void *dv, float *dg, float *dbeta,
                        float *dh0, void *workspace, size_t workspace_bytes, void *stream);

/* Which units run gdn_scan for this problem: 1 = matrix cores (bf16 MFMA
 * kernel), 0 = fp32 vector ALU kernel, -1 = invalid problem.  Lets callers
 * and benchmarks name the roofline that bounds the call. */
int32_t gdn_scan_backend(const gdn_problem *p);

/* Static description of a status code. */
const char *gdn_status_string(int32_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char *gdn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
