// kda_launch.h -- internal launchers behind the C ABI.  Arguments are
// already validated by kda_api.cpp; these only choose an instantiation and
// enqueue it.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

struct StepArgs {
    const void *q, *k, *v;
    const void *alpha;  // float32 decays, or logits in the dtype of q (fuse & 1)
    const float *beta;
    float *state;
    void *o;
    int N, H, dk, dv;
    bool bf16;
    int gate;  // kda_gate: 0 per channel, 1 per head, 2 none
    int fuse;  // kda_fuse_flag bits: 1 gate logits, 2 beta logits, 4 q/k L2 norm
    float scale;
};

hipError_t launch_recurrent_step(const StepArgs &a, hipStream_t stream);

struct ChunkArgs {
    const void *q, *k, *v;
    const void *alpha;  // float32 decays, or logits in the dtype of q (fuse & 1)
    const float *beta;
    const float *s0;
    void *o;
    float *sT;
    int B, T, H, dk, dv;
    bool bf16;
    int gate;               // kda_gate: 0 per channel, 1 per head, 2 none
    int fuse;               // kda_fuse_flag bits: 1 gate logits, 2 beta logits, 4 q/k L2 norm
    const int *cu_seqlens;  // device, NULL in dense mode
    int num_seqs;           // 0 in dense mode
    int *order;             // device workspace for the longest-first order (varlen), or NULL
    float scale;
    int dvt;                // value columns per workgroup (0 = choose)
    bool generic;           // bf16 through the generic kernel (A/B checks)
    float *ckpt = nullptr;  // chunk-start states for the backward (generic kernel), or NULL
    void *split_ws = nullptr;  // workspace of the two-segment path (chunk_split_plan), or NULL
};

hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t stream);

// Dense bf16 calls with few (sequence, head) units and long sequences run in
// two time segments at once (chunk_split.hip).  The plan: the first segment's
// tokens per sequence (a multiple of the chunk), the second's, and the
// workspace layout; bytes == 0 when the shape does not qualify.
struct SplitPlan {
    int l0 = 0, l1 = 0;
    size_t off_sm = 0, off_phi = 0, off_r = 0, off_z = 0, bytes = 0;
};
SplitPlan chunk_split_plan(int B, int T, int H, int dk, int dv);
// the chunk-wise forward in two time segments; ws holds chunk_split_plan().bytes
hipError_t launch_chunk_split(const ChunkArgs &a, void *ws, hipStream_t stream);

// Sequences a call of kda_chunk_fwd_noalloc may pack: the size of the device
// array that holds their order in place of a caller workspace.
constexpr int NOALLOC_MAX_SEQS = 65536;
// Device address of that array on the device of `stream` (looked up once per
// device, then reused).  Every call on one device shares the array.
hipError_t noalloc_order_buffer(hipStream_t stream, int **out);

// longest-first order of packed sequences into `order` (num_seqs ints)
hipError_t launch_order_sequences(const int *cu_seqlens, int num_seqs, int *order,
                                  hipStream_t stream);

// value-column tile the planner picks for a given number of units
int plan_chunk_dvt(int units, int dv, bool bf16);

// Gated DeltaNet-2: per-key-channel erase and write gates in place of beta
struct Gdn2StepArgs {
    const void *q, *k, *v;
    const float *alpha;          // [N, H, dk] decays, or NULL (no forget gate)
    const float *erase, *write;  // [N, H, dk]
    float *state;
    void *o;
    int N, H, dk, dv;
    bool bf16;
    float scale;
};

hipError_t launch_gdn2_step(const Gdn2StepArgs &a, hipStream_t stream);

struct Gdn2ChunkArgs {
    const void *q, *k, *v;
    const float *alpha;          // [B, T, H, dk] decays, or NULL (no forget gate)
    const float *erase, *write;  // [B, T, H, dk]
    const float *s0;
    void *o;
    float *sT;
    int B, T, H, dk, dv;
    bool bf16;
    const int *cu_seqlens;  // device, NULL in dense mode
    int num_seqs;
    int *order;             // device workspace for the longest-first order (varlen), or NULL
    float scale;
    int dvt;                // value columns per workgroup (0 = choose)
};

hipError_t launch_gdn2_chunk_fwd(const Gdn2ChunkArgs &a, hipStream_t stream);

struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *alpha, *beta, *s0, *dsT;
    float *g_q, *g_k, *g_v, *g_alpha, *g_beta, *g_s0;  // gradients
    int B, T, H, dk, dv;
    bool bf16;
    const int *cu_seqlens;  // device, NULL in dense mode
    int num_seqs;
    float scale;
    void *workspace;
};

// float32 inputs: the token recurrence run backwards over 8-token checkpoints
hipError_t launch_backward(const BwdArgs &a, hipStream_t stream);
// bf16 inputs: the chunk form (a forward pass storing chunk-start states, then
// the reverse sweep over chunks)
hipError_t launch_bwd_chunk(const BwdArgs &a, hipStream_t stream);

// Workspace layouts (kda_sizes.cpp, host code only).
// launch_backward: the state every 8 tokens of every unit
size_t backward_workspace_bytes(long tokens_total, int nseq, int H, int dk, int dv);
// launch_bwd_chunk: the state at every chunk start and end of every unit
// (bwd_chunk_ckpt_bytes, 256-byte multiple), then for each value-column slice
// but the first its partial dq, dk, dalpha and dbeta, the last padded to
// bwd_chunk_beta_rows floats
size_t bwd_chunk_ckpt_bytes(long tokens_total, int nseq, int H, int dk, int dv);
size_t bwd_chunk_beta_rows(long tokens_total, int H);
size_t bwd_chunk_workspace_bytes(long tokens_total, int nseq, int H, int dk, int dv);

}  // namespace kda
