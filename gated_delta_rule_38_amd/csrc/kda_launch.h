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
};

hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t stream);

// value-column tile the planner picks for a given number of units
int plan_chunk_dvt(int units, int dv, bool bf16);

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

hipError_t launch_backward(const BwdArgs &a, hipStream_t stream);
// workspace of launch_backward: the state checkpoints of every unit
size_t backward_workspace_bytes(long tokens_total, int nseq, int H, int dk, int dv);

}  // namespace kda
