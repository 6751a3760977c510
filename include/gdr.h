/*
 * gdr.h -- C ABI of libgdr.so: the chunkwise-parallel forward pass of the
 * gated delta-rule family of linear attention on AMD MI355X (gfx950), and the
 * backward pass of its KDA and gated DPLR forms.
 *
 * The operation (per sequence n and head h; "Diagonal Plus Low Rank" notes,
 * section 2, the original gated DPLR formula, with the write term scaled by
 * beta as in eq. 1 of "How to make GDN2 more stable"):
 *
 *     S = S0[n,h]                                   (dv x dk, zero if S0 == NULL)
 *     for each token t of the sequence, in order:
 *         S    = S Diag(alpha_t) (I - b_t a_t^T) + beta_t v_t k_t^T
 *         O[t] = S q_t
 *     S_final[n,h] = S
 *
 * alpha_t = exp(log_alpha) per key channel (GDR_GATE_CHANNEL), one value per
 * head (GDR_GATE_HEAD), or 1 (GDR_GATE_NONE).  With a == b == NULL the library
 * uses a = k, b = beta k: this is KDA (channel gate), Gated DeltaNet (head gate)
 * and DeltaNet (no gate) -- the special cases listed under "relation to KDA" in
 * the same notes.  With a and b given it is gated DPLR; pass beta = 1 for the
 * unscaled write term.
 *
 * The library evaluates this with the chunkwise rewrite of the pages: the UT
 * transform and WY factors inside each chunk of C tokens ("Kimi Delta
 * Attention backward" notes, forward recap; "DeltaNet" notes, section 4.1),
 * the triangular inverse of section 4.2 of the DeltaNet notes, and a serial
 * state pass across chunks.  Results equal the recurrence up to rounding.
 *
 * Memory: every tensor pointer is a DEVICE pointer to contiguous row-major,
 * 16-byte aligned memory owned by the caller.  The library allocates nothing, frees nothing
 * and keeps no pointer after a call returns.  All work is enqueued on
 * `stream` (a hipStream_t; NULL is the default stream) and the call returns
 * without synchronising: buffers must stay valid until that work completes.
 * Apart from the per-GPU scratch array of gdr_chunk_fwd_noalloc (see there), the
 * library keeps no state; concurrent calls on different streams with disjoint
 * outputs and workspaces are safe.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes.  Validation happens on the host before anything is enqueued,
 * so a non-zero code means no GPU work was launched (except GDR_ERR_HIP,
 * which reports a failed launch). */
typedef enum {
    GDR_OK = 0,
    GDR_ERR_NULL = -1,        /* a required pointer is NULL, or exactly one of a/b is NULL */
    GDR_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    GDR_ERR_UNSUPPORTED = -3, /* valid, but no kernel for this dtype/shape/chunk size */
    GDR_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than gdr_chunk_fwd_workspace() */
    GDR_ERR_ALIAS = -5,       /* O or S_final overlaps an input it must not overwrite */
    GDR_ERR_HIP = -6,         /* a HIP runtime call failed */
    GDR_ERR_ALIGN = -7        /* a tensor pointer or the workspace is not 16-byte aligned */
} gdr_status;

/* Element type of q, k, v, a, b and O.  log_alpha, beta, S0 and S_final are
 * always fp32. */
typedef enum { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

/* Gate layout. NONE: alpha = 1 (log_alpha must be NULL).  HEAD: log_alpha is
 * [tokens, H].  CHANNEL: log_alpha is [tokens, H, dk].
 *
 * GDR_GATE_CLIP may be OR-ed into any layout: the spectral clipping of the
 * forget gate from "How to make GDN2 more stable" (eq. 7).  Per token and head,
 * rho_t = ||I - b_t a_t^T||_2 (closed form of eq. 4, the vector norms moved into
 * eta: rho = (|a||b| + sqrt(|a|^2 |b|^2 - 4 a.b + 4)) / 2) and the gate becomes
 * alpha_t = min(alpha_t, 1 / rho_t) channel by channel before it is applied,
 * which bounds ||Diag(alpha_t)(I - b_t a_t^T)||_2 by 1 (eq. 2).  With
 * GDR_GATE_NONE the clipped gate is 1 / rho_t.  With a == b == NULL the factor is
 * a = k, b = beta k.  The clip is computed in fp32 from the input values. */
typedef enum {
    GDR_GATE_NONE = 0,
    GDR_GATE_HEAD = 1,
    GDR_GATE_CHANNEL = 2,
    GDR_GATE_CLIP = 4
} gdr_gate;

/* Bytes of device workspace gdr_chunk_fwd needs for these arguments (n_seq:
 * the number of packed sequences, or 0 without cu_seqlens; has_ab: non-zero
 * when a and b are given).  Returns 0 when the arguments are invalid
 * or unsupported.  The first 256 bytes of a workspace hold a sticky device
 * error flag (see gdr_workspace_error); zero-fill a workspace before its first
 * use.  The size depends on the current device's compute-unit count (with few
 * (sequence, head) pairs the serial pass is split across more CUs and needs
 * room for the partial states): query it for the device the call runs on. */
size_t gdr_chunk_fwd_workspace(int B, int H, int T, int dk, int dv, int C, int n_seq,
                               int dtype, int gate, int has_ab);

/* The forward pass.
 *
 *   q, k        [B, T, H, dk]  dtype          queries, keys
 *   v           [B, T, H, dv]  dtype          values
 *   a, b        [B, T, H, dk]  dtype or NULL  the rank-one factor I - b a^T
 *                                             (both NULL: a = k, b = beta k)
 *   log_alpha   see gdr_gate, fp32            log of the forget gate (<= 0 expected)
 *   gate        a gdr_gate layout, optionally | GDR_GATE_CLIP
 *   beta        [B, T, H]      fp32           write strength
 *   S0          [N, H, dv, dk] fp32 or NULL   initial state per sequence (NULL: zero)
 *   O           [B, T, H, dv]  dtype          output, o_t = S_t q_t
 *   S_final     [N, H, dv, dk] fp32 or NULL   final state per sequence
 *   cu_seqlens  [n_seq + 1]    int32 or NULL  packed sequences: sequence n is tokens
 *                                             [cu[n], cu[n+1]) of the B*T token axis;
 *                                             requires B == 1; N = n_seq.  Without it
 *                                             N = B and sequence n is batch row n.
 *               n_seq is ignored when cu_seqlens is NULL.
 *   C           chunk size (tokens per chunk).  The result does not depend on it
 *               beyond rounding.  Supported: 64 for bf16 without a, b; 16, 32 or
 *               64 for fp32 inputs and for bf16 with a, b (DPLR); and 128 for bf16
 *               without a, b at dk = 128 (each 128-token chunk's factors built from
 *               those of its two 64-token halves, "Gated Linear Attention" notes,
 *               section 5.3, secondary chunking; no log-domain rescue: a half whose
 *               gate falls by more than 2^192 in a channel raises error bit 2).
 *   dk, dv      head sizes; dk in {64, 128}; dv a multiple of 32 up to 256.
 *   Sizes: B, H, T >= 1, B * T * H * max(dk, dv) < 2^40 (elements of the largest
 *   tensor) and N * H < 2^27 ((sequence, head) pairs); otherwise GDR_ERR_SHAPE.
 *
 * S_final may equal S0 (in-place state update).  O must not overlap any input.
 * cu_seqlens lives in device memory and is not read on the host: malformed
 * offsets (decreasing, or beyond B*T) are clamped on the device, so no access
 * leaves the buffers, and raise the workspace error flag.  NaN or Inf inputs
 * propagate; they are not checked.
 */
int gdr_chunk_fwd(const void *q, const void *k, const void *v, const void *a, const void *b,
                  const float *log_alpha, const float *beta, const float *S0, void *O,
                  float *S_final, const int32_t *cu_seqlens, int n_seq, int B, int H, int T,
                  int dk, int dv, int C, int dtype, int gate, void *workspace,
                  size_t workspace_bytes, void *stream);

/* gdr_chunk_fwd for a training step: the same computation (the same O and
 * S_final, bit for bit), which also leaves in `workspace` the state entering
 * every chunk (bf16, where gdr_chunk_bwd reads it), so that the backward call
 * with GDR_BWD_FORWARD_STATES skips both its first kernel and its forward state
 * pass.  The state pass of the chunk form ("Kimi Delta Attention" notes,
 * forward recap; DPLR notes, section 2) already walks those states; storing
 * them costs the extra writes only.  Arguments and errors as gdr_chunk_fwd,
 * plus: the workspace must hold gdr_chunk_bwd_workspace bytes, and only what
 * gdr_chunk_bwd supports is accepted (else GDR_ERR_UNSUPPORTED; no gate
 * clipping). */
int gdr_chunk_fwd_for_bwd(const void *q, const void *k, const void *v, const void *a,
                          const void *b, const float *log_alpha, const float *beta,
                          const float *S0, void *O, float *S_final, const int32_t *cu_seqlens,
                          int n_seq, int B, int H, int T, int dk, int dv, int C, int dtype,
                          int gate, void *workspace, size_t workspace_bytes, void *stream);

/* Size of the fixed scratch array behind gdr_chunk_fwd_noalloc, per GPU (64 MiB). */
#define GDR_NOALLOC_SCRATCH_BYTES (64u << 20)

/* gdr_chunk_fwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The same kernels and the same results, bit for bit.
 * The workspace is a fixed device array of GDR_NOALLOC_SCRATCH_BYTES that every
 * GPU the library runs on holds from the first such call until the process
 * ends; the call itself allocates nothing (no hipMalloc, no library allocator).
 *
 *   q ... C, dtype, gate, stream   as for gdr_chunk_fwd
 *   flags   NULL, or a device int (4-byte aligned, owned by the caller) into which
 *           the call ORs the device error bits gdr_workspace_error would report
 *           (bit 1: malformed cu_seqlens were clamped); zero it before its first use
 *
 * Limits and errors: as gdr_chunk_fwd, plus GDR_ERR_WORKSPACE when the call would
 * need more than the array holds (gdr_chunk_fwd_workspace(...) >
 * GDR_NOALLOC_SCRATCH_BYTES; at dk = 128 roughly H * T <= 64K token-heads), and
 * GDR_ERR_HIP when the array's address cannot be obtained.  Every call on one GPU
 * uses that GPU's single array, which keeps the last call's contents: calls that
 * overlap in time on one GPU (on different streams, or from several threads
 * without ordering) race and give wrong results; serialise them on one stream. */
int gdr_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *a,
                          const void *b, const float *log_alpha, const float *beta,
                          const float *S0, void *O, float *S_final, const int32_t *cu_seqlens,
                          int n_seq, int B, int H, int T, int dk, int dv, int C, int dtype,
                          int gate, int *flags, void *stream);

/* Bytes of device workspace gdr_chunk_bwd needs (arguments as for
 * gdr_chunk_fwd_workspace).  Returns 0 when the arguments are invalid or
 * unsupported.  Zero-fill a workspace before its first use. */
size_t gdr_chunk_bwd_workspace(int B, int H, int T, int dk, int dv, int C, int n_seq, int dtype,
                               int gate, int has_ab);

/* Flags of gdr_chunk_bwd.
 *   GDR_BWD_FORWARD_WORKSPACE  `workspace` is the one a gdr_chunk_fwd call on the same
 *       q, k, v, a, b, log_alpha, beta, cu_seqlens, B, H, T, dk, dv, C and gate layout
 *       filled, enqueued earlier and followed by no other call on that workspace; its
 *       per-chunk factors are used instead of being recomputed (the forward's first
 *       kernel is skipped).  The workspace must still hold gdr_chunk_bwd_workspace
 *       bytes.  Nothing checks that the inputs are the same: when they differ the
 *       gradients are wrong.
 *   GDR_BWD_FORWARD_STATES  as GDR_BWD_FORWARD_WORKSPACE (implies it), for a workspace
 *       that gdr_chunk_fwd_for_bwd filled: its per-chunk states are used as well, and
 *       the backward's forward state pass is skipped. */
enum { GDR_BWD_FORWARD_WORKSPACE = 1, GDR_BWD_FORWARD_STATES = 2 };

/* The backward pass of gdr_chunk_fwd: the gradients of
 * L = <dO, O> + <dS_final, S_final> with respect to every input.  Without a, b
 * (KDA, Gated DeltaNet, DeltaNet) it follows the chunk-form backward of the
 * "Kimi Delta Attention backward" notes; with a, b the gated DPLR backward of the
 * "Diagonal Plus Low Rank" notes (section 3), beta scaling the write term as in
 * the forward.  A reverse serial pass over the chunks gives dL/dS, then each
 * chunk's gradients of the WY factors, the triangular inverse, beta and the gate.
 * The forward quantities it needs are recomputed from the inputs.
 *
 *   q, k, v, a, b, log_alpha, beta, S0, cu_seqlens, n_seq, B, H, T, dk, dv, C, gate
 *               as for gdr_chunk_fwd (gate: a layout; GDR_GATE_CLIP is unsupported)
 *   dO          [B, T, H, dv]  dtype          dL/dO
 *   dS_final    [N, H, dv, dk] fp32 or NULL   dL/dS_final (NULL: zero)
 *   dq, dk, dv  shapes of q, k, v, dtype      outputs
 *   da, db      shapes of a, b, dtype         outputs; NULL exactly when a, b are
 *   dlog_alpha  shape of log_alpha, fp32      output; NULL exactly when gate is NONE
 *   dbeta       [B, T, H]      fp32           output
 *   dS0         [N, H, dv, dk] fp32 or NULL   output dL/dS0
 *   flags       0, GDR_BWD_FORWARD_WORKSPACE or GDR_BWD_FORWARD_STATES (other bits:
 *               GDR_ERR_SHAPE)
 *
 * Supported: bf16, C = 64, dk in {64, 128}, dv a multiple of 32 up to 256.
 * Outputs may not overlap inputs, each other or the workspace.  Memory,
 * streams and errors as for gdr_chunk_fwd. */
int gdr_chunk_bwd(const void *q, const void *k, const void *v, const void *a, const void *b,
                  const float *log_alpha, const float *beta, const float *S0, const void *dO,
                  const float *dS_final, void *dq, void *dk, void *dv, void *da, void *db,
                  float *dlog_alpha, float *dbeta, float *dS0, const int32_t *cu_seqlens,
                  int n_seq, int B, int H, int T, int dk_, int dv_, int C, int dtype, int gate,
                  int flags, void *workspace, size_t workspace_bytes, void *stream);

/* Synchronises `stream`, returns the sticky device error flags of `workspace`
 * (0: none; bit 1: malformed cu_seqlens were clamped; bit 2: a chunk's gate falls
 * further than the kernels that ran can represent, so that call's results are
 * not valid -- gdr_chunk_bwd when a channel falls by more than 2^192 (e^133)
 * within a chunk, the fp32 kernels (fp32 inputs, or C < 64) by more than e^80, and the
 * bf16 forward with C = 128 when a 64-token half falls by more than 2^192; the bf16
 * forward with C = 64 handles such chunks in the log domain and never sets it) and
 * clears them.  Returns GDR_ERR_NULL or GDR_ERR_HIP on failure. */
int gdr_workspace_error(void *workspace, void *stream);

/* Human-readable text for a gdr_status value (static storage). */
const char *gdr_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
