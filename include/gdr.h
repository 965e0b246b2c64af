/*
 * gdr.h -- C ABI of libgdr, the gated delta rule on AMD Instinct MI355X (gfx950).
 *
 * The recurrence (column vectors, state S in R^{d_v x d_k}, stored row-major as S[v][c]):
 *
 *   scalar gate (Gated DeltaNet):   S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *   channel gate (KDA-style):       S_t = S_{t-1} Diag(a_t) (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *   output:                         o_t = S_t q_t   (read after the write)
 *
 * with a_t = exp(g_t): the library takes the LOG-decay g (g <= 0 for a decay in (0, 1]),
 * and b_t = beta_t.  Sources: "Linear Attention, Visualized" (snowchord.com), sections
 * "Recurrent form", "Gated DeltaNet (GDN)" and "Kimi Delta Attention (KDA)"; "Gated
 * DeltaNet: Householder Transitions and the Arithmetic of Forgetting" (mohakchugh.is-a.dev),
 * section "The gated delta rule".  The channel gate decays channel by channel first and then
 * applies the delta correction, as the KDA section states.
 *
 * No 1/sqrt(d) scale is applied (fold it into q), q and k are not normalised (the caller
 * L2-normalises keys, as the pages do by convention), and beta and g are not clamped.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers to contiguous row-major buffers owned by the
 *    caller.  The library allocates no device memory: the chunked entry points and
 *    gdr_frame_fwd take their scratch memory (the "workspace") from the caller, sized by the
 *    matching *_workspace_size query.  Between calls the library keeps only per-device launch
 *    settings, made on first use on each device: the dynamic LDS limit of its kernels and the
 *    device's compute-unit count.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue work and
 *    return; faults during execution surface at the caller's next synchronisation.
 *  - Every argument is validated on the host before anything is enqueued.  On any error the
 *    call returns a non-zero gdr_status and enqueues nothing.
 *  - Workspace: a device buffer of at least the queried size; its contents on entry are
 *    ignored and on return undefined; it may overlap no input or output.  A NULL, short or
 *    overlapping workspace returns GDR_ERR_WORKSPACE (a query result of 0 means none is
 *    needed and the argument is ignored).  Calls that share a workspace must be ordered on one
 *    stream.
 *  - io_dtype applies to q, k, v and o (GDR_BF16 or GDR_F32); g, beta and the state are
 *    always float32.
 *  - Supported sizes: d_k in {64, 128}; d_v a multiple of 32 in [32, 256].  With
 *    io_dtype = GDR_F32 the chunked forward supports d_k = 64 and the scalar gate only
 *    (GDR_ERR_UNSUPPORTED otherwise); decode supports every combination.
 *  - Numerics of the bf16 chunked forward: bf16 inputs are widened exactly; products run on
 *    fp16 MFMA with fp32 accumulation; the state is held in fp32 and rounded to an fp16
 *    operand copy once per 64-token chunk.  The state, the chunk's values and the terms
 *    derived from them (R, Z) are carried with a power-of-two scale chosen per chunk and per
 *    16 value channels, so their fp16 roundings do not depend on the overall scale of v and
 *    the initial state: the result scales exactly with (v, initial_state) while both stay
 *    inside fp32's range.  q, k and the gates enter fp16 operands unscaled, so |q|, |k|
 *    (and |k| times a per-channel decay factor) must stay below 65504.  o is rounded to bf16
 *    (RNE) once at the end.  The fp32-I/O forward and the decode step compute in fp32
 *    throughout.
 *  - Gates: the pages' gates decay, g <= 0 (0 < a <= 1), and the chunked kernels rely on it
 *    only for range: every decay factor they form is e^{G_i - G_j} with the later token i,
 *    at most 1.  A positive g is accepted and computed, but those factors then grow like
 *    e^{64 g} across a chunk (fp16 overflow past g of about 0.17 per token on average).
 *    beta (and the Gated DeltaNet-2 gates) are not clamped; the recurrence itself is
 *    contractive for unit keys with beta in [0, 2].
 *  - Non-finite inputs propagate: a NaN or infinity in one sequence's inputs affects that
 *    sequence's outputs and final state only.
  */
#ifndef GDR_H
#define GDR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdr_status {
    GDR_OK = 0,
    GDR_ERR_INVALID_ARG = 1, /* NULL where a buffer is required, negative size, bad enum  */
    GDR_ERR_SHAPE = 2,       /* a size outside the supported range                        */
    GDR_ERR_DTYPE = 3,       /* io_dtype is not GDR_BF16 or GDR_F32                       */
    GDR_ERR_UNSUPPORTED = 4, /* valid but not implemented combination                     */
    GDR_ERR_WORKSPACE = 5,   /* workspace NULL, smaller than required, or overlapping a buffer */
    GDR_ERR_HIP = 6          /* the HIP runtime rejected a launch                         */
} gdr_status;

typedef enum gdr_dtype { GDR_BF16 = 0, GDR_F32 = 1 } gdr_dtype;

typedef enum gdr_gate {
    GDR_GATE_SCALAR = 0,  /* g is [.., T] : one log-decay per token and head            */
    GDR_GATE_CHANNEL = 1  /* g is [.., T, d_k] : one log-decay per key channel (KDA)    */
} gdr_gate;

/* Library version as 10000*major + 100*minor + patch. */
int gdr_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *gdr_status_string(int status);

/*
 * gdr_chunk_fwd_workspace_size -- bytes of device workspace gdr_chunk_fwd needs.
 *
 * Per sequence and 64-token chunk the scalar gate takes 12864 bytes
 * (B*H*ceil(T/64)*12864) and the per-channel gate 12288 + 388 d_k bytes (61952 for d_k = 128,
 * 37120 for d_k = 64).  Returns 0 for GDR_F32 I/O (one kernel, no workspace), and -1 for sizes
 * or enums gdr_chunk_fwd would reject.
 */
int64_t gdr_chunk_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int d_k, int d_v,
                                     int io_dtype, int gate);

/*
 * gdr_chunk_fwd -- chunkwise-parallel forward pass over whole sequences.
 *
 * Computes, for each of the B*H independent (batch, head) sequences, every output o_t of
 * the recurrence above and the final state S_T, with the per-chunk algorithm of
 * "Linear Attention, Visualized", section "Gated DeltaNet (GDN)", "Complete per-chunk
 * algorithm" (scalar gate) and section "Reuse GLA and GDN" (channel gate), chunk size 64.
 * The page notes that the chunk-local quantities can be formed for all chunks in parallel
 * before the boundary pass threads the state through them; with bf16 I/O the call runs as
 * two kernels that do exactly that: the first forms, for every chunk at once,
 * T = N^{-1} diag(beta) (the UT transform, N = I + diag(beta) (Gam (.) K K^T)_strict) and the
 * decayed score matrix A, and writes them to the workspace; the second walks the chunks in
 * order with Z = T (V - diag(e^G) K S^T), O = diag(e^G) Q S^T + A Z and the state update.
 * With the per-channel gate (section "Kimi Delta Attention (KDA)") the first kernel also
 * writes the decayed copies K e^G, Q e^G, K e^{G_C - G} and e^{G_C}.  GDR_F32 I/O runs one
 * kernel with fp32 operands and needs no workspace.
 *
 *   q, k           [B, H, T, d_k]  io_dtype
 *   v              [B, H, T, d_v]  io_dtype
 *   g              [B, H, T] (GDR_GATE_SCALAR) or [B, H, T, d_k] (GDR_GATE_CHANNEL), float32
 *   beta           [B, H, T]       float32
 *   initial_state  [B, H, d_v, d_k] float32, or NULL for a zero state
 *   o              [B, H, T, d_v]  io_dtype, written (must not alias an input)
 *   final_state    [B, H, d_v, d_k] float32, written, or NULL to skip; may alias
 *                  initial_state exactly (each state tile is read before it is written)
 *   workspace      device buffer of at least gdr_chunk_fwd_workspace_size(...) bytes
 *                  (see the conventions above; GDR_ERR_WORKSPACE if missing or short)
 *   workspace_bytes  its size in bytes
 *
 * T may be any value in [0, 2^22] (a ragged last chunk is handled exactly; T = 0 copies
 * the initial state, or zeros, to final_state); a longer sequence returns GDR_ERR_SHAPE
 * (split it and carry the state).
 * B*H*T*max(d_k, d_v) must fit in int64.
 *
 * Per-channel gate: bf16 I/O only (GDR_ERR_UNSUPPORTED for GDR_F32).  Inside each 16-token
 * block the decay is factored through the block's 9th token while every channel's
 * log-decay stays within 6 of that token's; a wider block forms its diagonal 16x16 Gram tiles
 * afresh from the bf16 inputs with every factor of the form e^{G_i - G_j} (i the later token),
 * so any decay the fp32 gate can express is covered.
 */
gdr_status gdr_chunk_fwd(int64_t B, int64_t H, int64_t T, int d_k, int d_v,
                         int io_dtype, int gate,
                         const void *q, const void *k, const void *v,
                         const float *g, const float *beta,
                         const float *initial_state,
                         void *o, float *final_state,
                         void *workspace, int64_t workspace_bytes, void *stream);

/*
 * gdr_chunk_fwd_noalloc -- gdr_chunk_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same inputs, outputs, numerics and errors as gdr_chunk_fwd, without the workspace arguments:
 * the workspace is a device array inside the library, GDR_CHUNK_FWD_NOALLOC_WORKSPACE_BYTES
 * (96 MiB) on every GPU the library runs on, held from the library's load on that GPU until the
 * process ends.  The call allocates nothing (no hipMalloc, no library allocation).  A
 * configuration whose gdr_chunk_fwd_workspace_size exceeds that returns GDR_ERR_WORKSPACE
 * (the B=4, H=16, T=4096, d_k=d_v=128 scalar-gate shape needs 50.25 MiB and fits).
 *
 * All calls on one GPU share that GPU's array, which keeps the last call's contents (the
 * kernels need no particular contents on entry).  Calls that overlap on one GPU -- on
 * different streams, or from different threads without ordering -- race on the array and
 * give undefined results; order them on one stream.
 */
#define GDR_CHUNK_FWD_NOALLOC_WORKSPACE_BYTES (96u << 20)
gdr_status gdr_chunk_fwd_noalloc(int64_t B, int64_t H, int64_t T, int d_k, int d_v,
                                 int io_dtype, int gate,
                                 const void *q, const void *k, const void *v,
                                 const float *g, const float *beta,
                                 const float *initial_state,
                                 void *o, float *final_state, void *stream);

/*
 * gdr_chunk_fwd_fused_prep_workspace_size -- bytes of device workspace
 * gdr_chunk_fwd_fused_prep needs, per sequence and 64-token chunk, 13120 bytes (either d_k);
 * -1 for sizes gdr_chunk_fwd_fused_prep would reject.
 */
int64_t gdr_chunk_fwd_fused_prep_workspace_size(int64_t B, int64_t H, int64_t T, int d_k, int d_v);

/*
 * gdr_chunk_fwd_fused_prep -- gdr_chunk_fwd (scalar gate) from raw projections, with the
 * input preparation fused into the chunk kernels.
 *
 * Forms, per token and head, the inputs the recurrence assumes and runs the chunked forward
 * on them without writing q, k, g or beta out:
 *   q = q_raw / max(||q_raw||_2, 1e-6),  k = k_raw / max(||k_raw||_2, 1e-6)   (over d_k; the
 *       pages take keys L2-normalised by convention, and queries are treated the same way)
 *   beta = 1 / (1 + exp(-beta_logit))                                        (0 < beta < 1)
 *   g = log a = -exp(A_log[h]) * softplus(dt + dt_bias[h]),  softplus(x) = log(1 + e^x)
 * The gate is Mamba-2's construction ("Linear Attention, Visualized", section "Mamba-2:
 * input-dependent scalar decay", "Optional: Constructing the decay gate"): a decay rate
 * lambda = e^{A_log} per head times a positive step Delta_t = softplus(dt_t + b_Delta).
 * The first kernel normalises q and k (in fp32 before the fp16 rounding) for the chunk-local
 * products, forms beta and g, and writes T, A and the per-token factors of the state pass
 * with the inverse norms folded in (e^G / ||k||, e^{G_C - G} / ||k||, e^G / ||q||).  The
 * state kernel reads the raw q and k rows: every product it forms with them is scaled per
 * token, so the normalisation is exact there and no normalised row is ever written.
 *
 *   q_raw, k_raw     [B, H, T, d_k]  bf16 (not normalised)
 *   v                [B, H, T, d_v]  bf16
 *   dt, beta_logit   [B, H, T]       float32
 *   A_log, dt_bias   [H]             float32, one per head
 *   initial_state, o, final_state, workspace, workspace_bytes   as gdr_chunk_fwd
 *
 * Equivalent to computing q, k, g, beta as above and calling gdr_chunk_fwd with
 * GDR_GATE_SCALAR, except that q and k are not rounded to bf16 after the normalisation.
 * Range: the raw rows enter the state kernel's fp16 operands unscaled, so every element of
 * q_raw and k_raw must stay below 65504 in magnitude; rows whose elements all fall below
 * 6.1e-5 (fp16's smallest normal) lose accuracy there.
 * io_dtype must be GDR_BF16 (GDR_F32 returns GDR_ERR_UNSUPPORTED).  Sizes, T range and every
 * other error as for gdr_chunk_fwd.
 */
gdr_status gdr_chunk_fwd_fused_prep(int64_t B, int64_t H, int64_t T, int d_k, int d_v,
                                    int io_dtype,
                                    const void *q_raw, const void *k_raw, const void *v,
                                    const float *dt, const float *A_log, const float *dt_bias,
                                    const float *beta_logit,
                                    const float *initial_state,
                                    void *o, float *final_state,
                                    void *workspace, int64_t workspace_bytes, void *stream);

/*
 * gdr_gdp_chunk_fwd_workspace_size -- bytes of device workspace gdr_gdp_chunk_fwd needs:
 * the scalar gate's 12864 bytes per sequence and 64 virtual steps,
 * B*H*ceil(T*n_h/64)*12864; -1 for sizes gdr_gdp_chunk_fwd would reject.
 */
int64_t gdr_gdp_chunk_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int n_h, int d_k, int d_v);

/*
 * gdr_gdp_chunk_fwd -- chunkwise forward pass of the Gated Delta Product.
 *
 * "Linear Attention, Visualized", section "Gated Delta Product (GDP)": each token t carries
 * n_h substeps with their own key, value and beta.  The state decays once, by a_t = exp(g_t),
 * then takes the n_h updates in order,
 *     S <- S (I - b_{t,j} k_{t,j} k_{t,j}^T) + b_{t,j} v_{t,j} k_{t,j}^T,   j = 1..n_h,
 * and o_t = S q_t is read after the last one.  Computed, as that page's section "GDP as GDN
 * over a virtual sequence" describes, by the scalar-gate chunked forward of gdr_chunk_fwd run
 * over the T * n_h substeps in order (decay on each token's first substep, query and output
 * on its last), with the same numerics: the first kernel reads q_t on the last substep of a
 * token and g_t on its first, the state kernel writes o_t on the last substep.  n_h = 1 is
 * exactly gdr_chunk_fwd.
 *
 *   q              [B, H, T, d_k]         bf16
 *   k              [B, H, T, n_h, d_k]    bf16
 *   v              [B, H, T, n_h, d_v]    bf16
 *   g              [B, H, T]              float32, one log-decay per token
 *   beta           [B, H, T, n_h]         float32
 *   initial_state  [B, H, d_v, d_k] float32, or NULL for a zero state
 *   o              [B, H, T, d_v]         bf16, written (must not alias an input)
 *   final_state    [B, H, d_v, d_k] float32, written, or NULL; may alias initial_state exactly
 *   workspace, workspace_bytes   as gdr_chunk_fwd
 *
 * n_h in [1, 16] (n_h < 1: GDR_ERR_INVALID_ARG, n_h > 16: GDR_ERR_SHAPE); T * n_h <= 2^22
 * (GDR_ERR_SHAPE otherwise); io_dtype must be GDR_BF16 (GDR_F32 returns
 * GDR_ERR_UNSUPPORTED).  Sizes and every other error as for gdr_chunk_fwd.
 */
gdr_status gdr_gdp_chunk_fwd(int64_t B, int64_t H, int64_t T, int n_h, int d_k, int d_v,
                             int io_dtype,
                             const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             const float *initial_state,
                             void *o, float *final_state,
                             void *workspace, int64_t workspace_bytes, void *stream);

/*
 * gdr_gdn2_chunk_fwd_workspace_size -- bytes of device workspace gdr_gdn2_chunk_fwd needs:
 * gdr_chunk_fwd_workspace_size(B, H, T, d_k, d_v, GDR_BF16, GDR_GATE_CHANNEL) (-1 for sizes
 * gdr_gdn2_chunk_fwd would reject).
 */
int64_t gdr_gdn2_chunk_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int d_k, int d_v);

/*
 * gdr_gdn2_chunk_fwd -- chunkwise forward pass of Gated DeltaNet-2.
 *
 * "Gated DeltaNet-2, and the gate that was doing two jobs" (aigenapps.com), section 2: the
 * scalar beta of the delta rule splits into a key-side erase gate b_t and a value-side write
 * gate w_t, with KDA's per-channel decay a_t = exp(g_t):
 *     e_t = b_t (.) k_t,   z_t = w_t (.) v_t,
 *     S_t = S_{t-1} Diag(a_t) (I - e_t k_t^T) + z_t k_t^T,     o_t = S_t q_t
 * (the page's P_t = (I - k_t e_t^T) D_t P_{t-1} + k_t z_t^T for P = S^T): the decayed state is
 * read along e_t and the correction z_t - S Diag(a_t) e_t is written along k_t.  b = w = beta
 * on every channel is exactly gdr_chunk_fwd with GDR_GATE_CHANNEL.  Runs the per-channel-gate
 * two-kernel path: the first kernel forms, for every chunk at once, T = N^{-1} with the erase
 * gate in N's rows, A, and the decayed copies (b (.) k) e^G, q e^G, k e^{G_C - G}; the second
 * walks the chunks in order with Z = T (z - ((b (.) k) e^G) S^T), where z = w (.) v is formed
 * and kept in fp32.  Same numerics and decay coverage as the per-channel gate.
 *
 *   q, k           [B, H, T, d_k]  bf16
 *   v              [B, H, T, d_v]  bf16
 *   g              [B, H, T, d_k]  float32, per-channel log-decay
 *   b              [B, H, T, d_k]  float32, erase gate (the page uses [0, 1]; not clamped)
 *   w              [B, H, T, d_v]  float32, write gate (the page uses [0, 1]; not clamped)
 *   initial_state  [B, H, d_v, d_k] float32, or NULL for a zero state
 *   o              [B, H, T, d_v]  bf16, written (must not alias an input)
 *   final_state    [B, H, d_v, d_k] float32, written, or NULL; may alias initial_state exactly
 *   workspace, workspace_bytes   as gdr_chunk_fwd
 *
 * io_dtype must be GDR_BF16 (GDR_F32 returns GDR_ERR_UNSUPPORTED).  (T + 64) * d_v <= 2^30
 * (the fp32 write gate's 32-bit offsets), GDR_ERR_SHAPE otherwise.  Sizes, the rest of the T range and every other error as for gdr_chunk_fwd.
 */
gdr_status gdr_gdn2_chunk_fwd(int64_t B, int64_t H, int64_t T, int d_k, int d_v,
                              int io_dtype,
                              const void *q, const void *k, const void *v,
                              const float *g, const float *b, const float *w,
                              const float *initial_state,
                              void *o, float *final_state,
                              void *workspace, int64_t workspace_bytes, void *stream);

/*
 * gdr_frame_fwd -- the frame-level implicit update (tokens in unordered frames).
 *
 * The video delta-rule post (haoyizhu.site, "video-delta-rule"), section "A Different Route":
 * the sequence is cut into frames of frame_len tokens (the last frame may be shorter), and a
 * frame moves the state by one implicit gradient step on its total loss,
 *     G_t = K_t^T Gamma_t K_t,   C_t = V_t^T Gamma_t K_t,
 *     S_t (I + G_t) = S_{t-1} D_t + C_t,      o_i = S_t q_i for every token i of frame t,
 * with Gamma_t = diag(gamma) the tokens' writing strengths (gamma >= 0; the post's gamma =
 * s e^z) and D_t = exp(g_t) the frame's forget gate (scalar or per key channel), applied to
 * the old state first.  Every query of a frame reads the frame's final state, so the result
 * does not depend on the order of the tokens inside a frame.  With frame_len = 1 this is the
 * delta rule with beta = gamma / (1 + gamma) (but frame_len must be a multiple of 16 here).
 *
 *   q, k           [B, H, T, d_k]   bf16 (keys unit-norm by the pages' convention; not checked)
 *   v              [B, H, T, d_v]   bf16
 *   gamma          [B, H, T]        float32, >= 0
 *   g              [B, H, F] (GDR_GATE_SCALAR) or [B, H, F, d_k] (GDR_GATE_CHANNEL), float32,
 *                  F = ceil(T / frame_len): the log forget gate of each frame
 *   initial_state, o, final_state   as gdr_chunk_fwd
 *   workspace      device buffer of at least gdr_frame_fwd_workspace_size(...) bytes (per
 *                  sequence and frame: (I + G)^{-1} as two fp16 matrices, C in fp32 and the
 *                  frame's state in fp16 with one power-of-two exponent per 16 value channels),
 *                  owned by the caller, overlapping nothing else
 *
 * Supported: bf16 I/O, d_k and d_v in {64, 128} (GDR_ERR_UNSUPPORTED otherwise); frame_len a
 * positive multiple of 16 and (ceil(T / frame_len) + 1) * d_v * d_k * 4 < 2^32 (the state
 * pass addresses one sequence's per-frame records with 32-bit offsets; GDR_ERR_SHAPE
 * otherwise); T in [0, 2^22].  A NULL, short or overlapping workspace returns
 * GDR_ERR_WORKSPACE.  Numerics: G and C from fp16 MFMA operands
 * sqrt(gamma) k, sqrt(gamma) v with fp32 accumulation; (I + G)^{-1} by Gauss-Jordan
 * elimination in fp32; the state chained in fp32 with split-fp16 products, the right-hand
 * side D S + C scaled by a power of two per frame before its fp16 split; o from an fp16 copy
 * of each frame's state (scaled by a power of two per frame and 16 value channels), rounded
 * to bf16.  G and C must stay inside fp32's range, and sqrt(gamma) |k|, sqrt(gamma) |v| below
 * 65504.
 */
int64_t gdr_frame_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int frame_len, int d_k,
                                     int d_v);
gdr_status gdr_frame_fwd(int64_t B, int64_t H, int64_t T, int frame_len, int d_k, int d_v,
                         int io_dtype, int gate,
                         const void *q, const void *k, const void *v,
                         const float *gamma, const float *g,
                         const float *initial_state,
                         void *o, float *final_state,
                         void *workspace, int64_t workspace_bytes, void *stream);

/*
 * gdr_decode_step -- one recurrent token per sequence, state updated in place.
 *
 * One step of the recurrence ("Linear Attention, Visualized", section "Recurrent form",
 * with the decay of section "Gated DeltaNet (GDN)" or "Kimi Delta Attention (KDA)") for
 * N*H resident states, in a single pass over each state: decay, predict p = S k,
 * u = beta (v - p), S += u k^T, o = S q.
 *
 *   q, k   [N, H, d_k]   io_dtype
 *   v      [N, H, d_v]   io_dtype
 *   g      [N, H] (GDR_GATE_SCALAR) or [N, H, d_k] (GDR_GATE_CHANNEL), float32
 *   beta   [N, H]        float32
 *   state  [N, H, d_v, d_k] float32, read and overwritten in place
 *   o      [N, H, d_v]   io_dtype, written (must not alias the state or an input)
 *
 * N = 0 or H = 0 is a valid no-op.
 */
gdr_status gdr_decode_step(int64_t N, int64_t H, int d_k, int d_v,
                           int io_dtype, int gate,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           float *state, void *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
