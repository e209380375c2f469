/*
 * kda.h -- C ABI of libkda: the Kimi Delta Attention (KDA) gated delta-rule
 * recurrence on AMD Instinct MI355X (gfx950).
 *
 * The method.  Per independent unit (one batch entry or packed sequence, one
 * head) the state S is a dk x dv fp32 matrix (row = key channel, column =
 * value channel).  For each token t in order:
 *   forget   S~  = Diag(alpha_t) S_{t-1}          alpha_t in (0,1]^dk
 *   predict  vh  = S~^T k_t
 *   write    S_t = S~ + beta_t k_t (v_t - vh)^T   beta_t scalar per token/head
 *   read     o_t = scale * S_t^T q_t              scale = dk^{-1/2} by default
 * Source: "Kimi Delta Attention" (daiw.net, Kimi K3 manual), section
 * "KDA 的更新式" (the update S_t = (I - beta k k^T) Diag(alpha) S_{t-1}
 * + beta k v^T) and sections "一" (per-channel alpha) and "二" (delta rule);
 * bugfactory.tech news 3610, second to fourth paragraphs (the order forget,
 * predict, correct, write, read, and the dk^{-1/2} read scale).  The fifth
 * paragraph there names the two compute modes exposed here: a chunk-wise mode
 * for training and long contexts, and a token-by-token recurrent mode for
 * decoding.
 *
 * Conventions shared by every entry point:
 *  - Memory.  All tensor pointers are DEVICE pointers owned by the caller;
 *    tensors are dense, row-major (last index fastest).  Alignment: the
 *    chunk-wise q, k and alpha 8 bytes (read in pairs), the decode state 16
 *    bytes (read as float4), every other pointer its element size.  The
 *    library keeps no state between calls and allocates no device memory.
 *  - Streams.  Work is enqueued on `stream` (0 = the null stream) and the
 *    call returns without synchronising.  A launch failure returns
 *    KDA_ERROR_HIP; faults inside a kernel surface at the caller's next
 *    synchronisation.
 *  - Errors.  Arguments are validated on the host before anything is
 *    enqueued; on any error nothing is launched and no output is touched.
 *    The library never prints, throws across the ABI or aborts.
 *  - Thread safety.  Entry points are reentrant.
 *  - Supported shapes.  dk, dv in {64, 128}; chunk_size == 64.
 *  - Numerical domain.  Any alpha in [0, 1] (alpha = 1 is exact: DeltaNet).
 *    The chunk-wise kernels scale keys and queries by cumulative decays
 *    referenced to the middle of each 64-token chunk; a chunk whose product
 *    of alpha over either half falls below 2^-100 in some key channel would
 *    leave fp32's range there, so the kernel flags it and recomputes that
 *    (sequence, head, value-column slice) token by token at the end of the
 *    same launch, exactly and without ratios of decays.  Such work items run
 *    one token per step (tens of times slower); the others are unaffected.
 *    kda_backward (bf16) takes the token path from the last chunk whose
 *    half-chunk product is below 2^-12 back to the sequence start: the chunk
 *    form's decay gradient loses accuracy to cancellation as the decay across
 *    a chunk grows.  The recurrent steps have no such case.  NaN/Inf
 *    propagate.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_SUCCESS = 0,
    KDA_ERROR_INVALID_VALUE = 1,          /* null pointer, negative size, bad cu_seqlens, overlap */
    KDA_ERROR_NOT_SUPPORTED = 2,          /* dk/dv/chunk_size outside the supported set */
    KDA_ERROR_MISALIGNED = 3,             /* a pointer breaks the alignment rules above */
    KDA_ERROR_INSUFFICIENT_WORKSPACE = 4, /* workspace smaller than kda_chunk_fwd_workspace_size() */
    KDA_ERROR_HIP = 5                     /* the HIP runtime rejected a launch */
} kda_status;

typedef enum {
    KDA_DTYPE_F32 = 0,  /* q, k, v and o are float32 */
    KDA_DTYPE_BF16 = 1  /* q, k, v and o are bfloat16; o is rounded to nearest even */
} kda_dtype;

/*
 * Granularity of the forget gate alpha (the *_gated entry points).
 * KDA_GATE_CHANNEL: one decay per token, head and key channel, Diag(alpha_t)
 *   ("Kimi Delta Attention", section "一、Diag(α_t)：通道级遗忘").
 * KDA_GATE_HEAD: one decay per token and head, alpha_t S_{t-1} for the whole
 *   state: Gated DeltaNet (bugfactory.tech news 3610, third paragraph; the
 *   per-head scalar rows of the table in the same section of "Kimi Delta
 *   Attention").  Equal to KDA_GATE_CHANNEL with alpha_t repeated over the
 *   dk channels.
 * KDA_GATE_NONE: no forget gate, alpha = 1: DeltaNet (bugfactory.tech news
 *   3610, second paragraph).  alpha must be NULL.
 */
typedef enum {
    KDA_GATE_CHANNEL = 0, /* alpha [.., H, dk] float32 */
    KDA_GATE_HEAD = 1,    /* alpha [.., H] float32 */
    KDA_GATE_NONE = 2     /* alpha == NULL */
} kda_gate;

/*
 * In-kernel preparation of the inputs (flags of the *_fused entry points),
 * so that the raw outputs of the projections that produce them need no
 * separate pass over HBM:
 * KDA_FUSE_GATE_LOGITS: `gate` holds logits z in the dtype of q (bf16 or
 *   float32) and the decay is alpha = sigmoid(z) = 1 / (1 + exp(-z)),
 *   evaluated in float32 as 1 / (1 + 2^(-z log2 e)), which keeps alpha in
 *   (0, 1) as the per-channel decay of "Kimi Delta Attention", section
 *   "一、Diag(α_t)：通道级遗忘" requires.  Without the flag `gate` holds
 *   alpha itself in float32.
 * KDA_FUSE_BETA_LOGITS: `beta` holds logits b (float32) and the write
 *   strength is beta = sigmoid(b), in (0, 1) (the data-dependent update
 *   strength listed under "在DeltaNet基础上的进一步演进" on the kongchang.com
 *   page).
 * KDA_FUSE_QK_L2NORM: q and k are divided by their L2 norm per token and
 *   head, x / sqrt(sum x^2 + 1e-6), in float32 before any other use (with
 *   unit keys, beta = 1 makes the write an exact overwrite: bugfactory.tech
 *   news 3610, second paragraph).
 */
typedef enum {
    KDA_FUSE_GATE_LOGITS = 1,
    KDA_FUSE_BETA_LOGITS = 2,
    KDA_FUSE_QK_L2NORM = 4
} kda_fuse_flag;

/*
 * Device workspace (bytes) that kda_chunk_fwd needs.  Dense calls
 * (num_seqs == 0) need none; packed variable-length calls need 4 bytes per
 * sequence (rounded up to 256), used to order sequences longest first.
 * Returns 0 for arguments kda_chunk_fwd would reject.
 */
size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int num_seqs,
                                    kda_dtype dtype);

/*
 * Device workspace (bytes) with which a dense bf16 call of kda_chunk_fwd,
 * kda_chunk_fwd_gated or kda_chunk_fwd_fused runs each sequence in two time
 * segments at once; 0 when the shape does not qualify (it needs
 * dk = dv = 128, at most 32 (batch, head) units and T >= 4033, i.e. at least
 * 64 chunks).
 * Source: the update of "Kimi Delta Attention", section "KDA 的更新式", is
 * affine in the state, so the second segment's states are Phi_t X + R_t for
 * the unknown start X, and the chunk-parallel state passing of the
 * kongchang.com page, section "硬件效率的优化策略", then applies inside one
 * sequence: the first segment (from initial_state) and the second segment's
 * transition part Phi (from the identity, zero values) and zero-start part R
 * run concurrently (two more streams of the library's own, forked from and
 * joined back to `stream` with events), and a last pass forms
 * o_t = o^R_t + Sm^T z_t and the final state Phi_T Sm + R_T from the first
 * segment's final state Sm.
 * A call whose workspace holds at least this many bytes, 256-byte aligned,
 * with o 8-byte aligned, takes that path; otherwise (and for
 * kda_chunk_fwd_noalloc) the single pass.
 * The two agree up to rounding (z_t = scale Phi_t^T q_t is kept in bf16, Sm
 * enters the output products as two bf16 parts with fp32 accumulation); each
 * is deterministic.  Concurrent calls on one device share those streams and
 * serialise their second-segment kernels on them.
 */
size_t kda_chunk_fwd_split_workspace_size(int B, int T, int H, int dk, int dv, kda_dtype dtype);

/*
 * Chunk-wise forward (64-token chunks) over whole sequences.
 * Source: the chunk-wise mode of bugfactory.tech news 3610, fifth paragraph,
 * and the chunk-parallel scheme on the kongchang.com page, section
 * "硬件效率的优化策略" (matrix products inside a chunk, the state carried
 * between chunks).
 *
 * Dense mode (cu_seqlens_dev == NULL, num_seqs == 0):
 *   q, k    [B, T, H, dk]  dtype
 *   v, o    [B, T, H, dv]  dtype        (o is written)
 *   alpha   [B, T, H, dk]  float32
 *   beta    [B, T, H]      float32
 *   initial_state, final_state  [B, H, dk, dv] float32
 * Packed variable-length mode (num_seqs >= 1, B == 1):
 *   sequence n occupies tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 of the
 *   T = cu_seqlens[num_seqs] packed tokens; states are [num_seqs, H, dk, dv].
 *   cu_seqlens_dev (device) and cu_seqlens_host (host) hold the same
 *   num_seqs + 1 non-decreasing int32 offsets starting at 0; the host copy is
 *   used for validation and launch planning without a device sync.
 *   Empty sequences are allowed (final = initial).
 * initial_state == NULL means a zero start.  final_state == NULL skips the
 * state store.  initial_state == final_state updates the state in place.
 * scale <= 0 selects dk^{-1/2}.  chunk_size must be 64.
 * workspace: device memory of at least kda_chunk_fwd_workspace_size() bytes
 * (may be NULL when that is 0).  Outputs must not overlap inputs except for
 * the in-place state.
 */
kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, const float *alpha,
                         const float *beta, const float *initial_state, void *o,
                         float *final_state, int B, int T, int H, int dk, int dv,
                         kda_dtype dtype, const int *cu_seqlens_dev,
                         const int *cu_seqlens_host, int num_seqs, float scale,
                         int chunk_size, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * kda_chunk_fwd with the forget gate's granularity chosen by `gate`: alpha is
 * [B, T, H, dk] (KDA_GATE_CHANNEL, the same call as kda_chunk_fwd),
 * [B, T, H] (KDA_GATE_HEAD) or NULL (KDA_GATE_NONE); a per-head alpha needs
 * 4-byte alignment.  Every other argument, the layouts, the aliasing rules
 * and the errors are those of kda_chunk_fwd; a gate outside the enum, or an
 * alpha that is NULL where one is needed (or not NULL for KDA_GATE_NONE),
 * returns KDA_ERROR_INVALID_VALUE.
 */
kda_status kda_chunk_fwd_gated(const void *q, const void *k, const void *v, const float *alpha,
                               const float *beta, const float *initial_state, void *o,
                               float *final_state, int B, int T, int H, int dk, int dv,
                               kda_dtype dtype, kda_gate gate, const int *cu_seqlens_dev,
                               const int *cu_seqlens_host, int num_seqs, float scale,
                               int chunk_size, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * kda_chunk_fwd_gated with in-kernel input preparation: `flags` is a bitwise
 * OR of kda_fuse_flag values (0 gives kda_chunk_fwd_gated exactly).  With
 * KDA_FUSE_GATE_LOGITS, `gate` has the shape of alpha for `gate_kind` and the
 * dtype of q; without it, `gate` is the float32 alpha.  KDA_GATE_NONE takes
 * gate == NULL and no KDA_FUSE_GATE_LOGITS.  Alignment: q, k and a
 * per-channel gate 8 bytes, a per-head gate its element size.  Errors as
 * for kda_chunk_fwd_gated, plus KDA_ERROR_INVALID_VALUE for unknown flags.
 */
kda_status kda_chunk_fwd_fused(const void *q, const void *k, const void *v, const void *gate,
                               const float *beta, const float *initial_state, void *o,
                               float *final_state, int B, int T, int H, int dk, int dv,
                               kda_dtype dtype, kda_gate gate_kind, unsigned flags,
                               const int *cu_seqlens_dev, const int *cu_seqlens_host,
                               int num_seqs, float scale, int chunk_size, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, and the same results bit for bit
 * as kda_chunk_fwd's single pass (a dense call that takes kda_chunk_fwd's
 * two-segment path, see kda_chunk_fwd_split_workspace_size, agrees with it up
 * to rounding).  It calls no hipMalloc, hipFree or allocating library routine.  The only
 * scratch, the longest-first order of the packed sequences, lives in a
 * fixed device array of KDA_NOALLOC_MAX_SEQS ints (256 KiB) that each GPU
 * the library runs on holds until the process ends; the order is rewritten
 * in full by every variable-length call, and dense calls do not use it.
 * Errors as for kda_chunk_fwd, plus KDA_ERROR_NOT_SUPPORTED for
 * num_seqs > KDA_NOALLOC_MAX_SEQS (nothing is launched).  Every call on one
 * GPU shares that array: variable-length calls that overlap in time on one
 * GPU (on different streams, or from different threads) race on it and must
 * be ordered by the caller.
 */
#define KDA_NOALLOC_MAX_SEQS 65536
kda_status kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                 const float *alpha, const float *beta,
                                 const float *initial_state, void *o, float *final_state, int B,
                                 int T, int H, int dk, int dv, kda_dtype dtype,
                                 const int *cu_seqlens_dev, const int *cu_seqlens_host,
                                 int num_seqs, float scale, int chunk_size, hipStream_t stream);

/*
 * One decode step, state updated in place.
 * Source: the fused recurrent mode of bugfactory.tech news 3610, fifth
 * paragraph (the sequence is processed token by token, state tiles updated
 * independently per batch entry and head); one call is one token.
 *   q, k   [N, H, dk]  dtype
 *   v, o   [N, H, dv]  dtype     (o is written)
 *   alpha  [N, H, dk]  float32
 *   beta   [N, H]      float32
 *   state  [N, H, dk, dv] float32, read and rewritten
 * scale <= 0 selects dk^{-1/2}.  o must not overlap state or the inputs.
 */
kda_status kda_recurrent_step(const void *q, const void *k, const void *v, const float *alpha,
                              const float *beta, float *state, void *o, int N, int H, int dk,
                              int dv, kda_dtype dtype, float scale, hipStream_t stream);

/*
 * kda_recurrent_step with the forget gate's granularity chosen by `gate`:
 * alpha is [N, H, dk] (KDA_GATE_CHANNEL, the same call as
 * kda_recurrent_step), [N, H] (KDA_GATE_HEAD) or NULL (KDA_GATE_NONE).
 * Errors as for kda_recurrent_step, plus KDA_ERROR_INVALID_VALUE for a gate
 * outside the enum or an alpha that does not match it.
 */
kda_status kda_recurrent_step_gated(const void *q, const void *k, const void *v,
                                    const float *alpha, const float *beta, float *state,
                                    void *o, int N, int H, int dk, int dv, kda_dtype dtype,
                                    kda_gate gate, float scale, hipStream_t stream);

/*
 * kda_recurrent_step_gated with in-kernel input preparation: `flags` and
 * `gate` as for kda_chunk_fwd_fused ([N, H, dk], [N, H] or NULL).
 */
kda_status kda_recurrent_step_fused(const void *q, const void *k, const void *v,
                                    const void *gate, const float *beta, float *state, void *o,
                                    int N, int H, int dk, int dv, kda_dtype dtype,
                                    kda_gate gate_kind, unsigned flags, float scale,
                                    hipStream_t stream);

/*
 * Device workspace (bytes) that kda_backward needs.  bf16: the float32
 * state of every (sequence, head) at the start of every 64-token chunk and
 * after the last, (tokens/64 + 2 * sequences + 1) * H * dk * dv * 4 bytes
 * rounded up to 256, then the partial gradients of value-column slices 1 ..
 * dv/32 - 1, (dv/32 - 1) * (3 * tokens * H * dk + tokens * H rounded up to
 * 64) * 4 bytes.  float32: a state checkpoint every 8 tokens, (tokens/8
 * rounded up + sequences + 1) * H * dk * dv * 4 bytes rounded up to 256.
 * Returns 0 for arguments kda_backward would reject.
 */
size_t kda_backward_workspace_size(int B, int T, int H, int dk, int dv, int num_seqs,
                                   kda_dtype dtype);

/*
 * Gradients of kda_chunk_fwd (per-channel gate, no input preparation): given
 * dout = dL/do and dfinal_state = dL/dS_T, returns dL/dq, dL/dk, dL/dv,
 * dL/dalpha, dL/dbeta and dL/dS_0.
 * Source: the chain rule through the four steps of the update ("Kimi Delta
 * Attention", section "KDA 的更新式"; bugfactory.tech news 3610, second to
 * fourth paragraphs); the fifth paragraph there names training as the use of
 * the chunk-wise mode.  bf16 inputs: a chunk-wise forward stores the state at
 * every chunk start, then a reverse sweep over chunks applies the chain rule
 * to the chunk form on the matrix cores (bf16 operands, fp32 accumulation;
 * see the numerical domain above for the chunks it takes token by token).
 * float32 inputs: the token recurrence run backwards from 8-token
 * checkpoints, in fp32.
 *   q, k, v, alpha, beta, initial_state, B, T, H, dk, dv, dtype, cu_seqlens_*,
 *   num_seqs, scale: as for kda_chunk_fwd (the forward being differentiated)
 *   dout          [B, T, H, dv]  dtype
 *   dfinal_state  [Ns, H, dk, dv] float32, or NULL (zero)
 *   dq, dk        [B, T, H, dk]  float32 (written)
 *   dv            [B, T, H, dv]  float32 (written)
 *   dalpha        [B, T, H, dk]  float32 (written)
 *   dbeta         [B, T, H]      float32 (written)
 *   dinitial_state [Ns, H, dk, dv] float32 (written; required)
 * The states and their gradients need 16-byte alignment, v and dout four
 * times their element size (8 bytes for bf16, 16 for float32), the other
 * tensors their element size.  workspace: device memory of at least
 * kda_backward_workspace_size() bytes, 256-byte aligned.  Outputs must not
 * overlap inputs, each other or the workspace.  Errors as for kda_chunk_fwd.
 * T == 0 (or varlen with every sequence empty) is valid: dinitial_state is
 * then dfinal_state (zero if NULL).
 * Determinism: bf16 gradients are bitwise reproducible (each of the dv/32
 * value-column slices of a unit writes its part of dq, dk, dalpha and dbeta
 * into a workspace plane of its own, and the planes are added in slice
 * order).  float32: dv and dinitial_state are reproducible; dq, dk, dalpha
 * and dbeta sum the dv/16 slices' parts with float atomics, so their last
 * bits can differ from run to run.
 */
kda_status kda_backward(const void *q, const void *k, const void *v, const float *alpha,
                        const float *beta, const float *initial_state, const void *dout,
                        const float *dfinal_state, float *dq, float *dk, float *dv,
                        float *dalpha, float *dbeta, float *dinitial_state, int B, int T, int H,
                        int dk_dim, int dv_dim, kda_dtype dtype, const int *cu_seqlens_dev,
                        const int *cu_seqlens_host, int num_seqs, float scale, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * Gated DeltaNet-2 ("线性注意力机制：从标准注意力到 Gated DeltaNet-2",
 * jindou-blog, section 4 "Gated DeltaNet-2：解耦擦除与写入"): the delta rule's
 * one write strength beta is split into an erase gate e_t and a write gate
 * w_t, each one value per key channel, with KDA's per-channel forget gate
 * kept.  Per token (the page prints the update garbled; this is the reading
 * under which KDA, Gated DeltaNet and linear attention are its special cases,
 * as the page's table states):
 *   forget  S~  = Diag(alpha_t) S_{t-1}
 *   predict vh  = S~^T k_t
 *   erase   S'  = S~ - (e_t . k_t) vh^T        ((e . k)_i = e_i k_i)
 *   write   S_t = S' + (w_t . k_t) v_t^T
 *   read    o_t = scale * S_t^T q_t
 * e_t = w_t = beta_t is KDA exactly; e_t = 0 is a gated linear attention.
 *
 * kda_gdn2_chunk_fwd: the chunk-wise forward; arguments as for
 * kda_chunk_fwd, with erase and write [B, T, H, dk] float32 in place of beta,
 * and alpha [B, T, H, dk] float32 or NULL (no forget gate, alpha = 1).
 * q, k, alpha, erase and write need 8-byte alignment.  Only bf16 q, k, v
 * (dtype KDA_DTYPE_BF16) are supported (KDA_ERROR_NOT_SUPPORTED otherwise).
 * workspace as for kda_chunk_fwd (kda_chunk_fwd_workspace_size).  The decay
 * domain is that of kda_chunk_fwd.
 */
kda_status kda_gdn2_chunk_fwd(const void *q, const void *k, const void *v, const float *alpha,
                              const float *erase, const float *write,
                              const float *initial_state, void *o, float *final_state, int B,
                              int T, int H, int dk, int dv, kda_dtype dtype,
                              const int *cu_seqlens_dev, const int *cu_seqlens_host,
                              int num_seqs, float scale, int chunk_size, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * kda_gdn2_recurrent_step: one Gated DeltaNet-2 decode step, state updated in
 * place; arguments as for kda_recurrent_step with erase and write [N, H, dk]
 * float32 in place of beta and alpha [N, H, dk] float32 or NULL.  bf16 and
 * float32 q, k, v are supported, and any alpha in (0, 1] (the step takes no
 * running products).
 */
kda_status kda_gdn2_recurrent_step(const void *q, const void *k, const void *v,
                                   const float *alpha, const float *erase, const float *write,
                                   float *state, void *o, int N, int H, int dk, int dv,
                                   kda_dtype dtype, float scale, hipStream_t stream);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char *kda_status_string(kda_status status);

/* Library version as major*10000 + minor*100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
