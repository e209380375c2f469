// chunk_common.h -- pieces shared by the chunk-wise forward kernels: kernel
// parameters, the XCD-aware work-item mapping and small LDS helpers.
#pragma once

#include "kda_device.h"
#include "kda_launch.h"

#include <type_traits>

namespace kda {

constexpr int CH = 64;  // chunk length

struct KParams {
    const void *q, *k, *v;
    const void *alpha;  // float32 decays, or logits in the dtype of q (FUSE_GATE_LOGITS)
    const float *beta, *s0;
    void *o;
    float *sT;
    const int *cu_seqlens;
    const int *order;
    int B, T, H, dv, units, njt_all;
    int gate;  // 0: alpha per key channel, 1: per head (Gated DeltaNet), 2: none (alpha = 1)
    int fuse;  // kda_fuse_flag bits (FUSE_*)
    float scale;
    // the state at the start of every chunk and after the last one, for the
    // chunk-form backward (slots as laid out in chunk_fwd.hip), or NULL
    float *ckpt = nullptr;
    // dense calls: tokens taken from each sequence, the first t_len of its T
    // rows from the base pointers (-1: all T)
    int t_len = -1;
    // the transition part of a time segment: the same recurrence started from
    // the identity (dv == dk) with every value read as zero (s0 unused)
    bool ident = false;
};

struct WorkItem {
    bool valid;
    int h, seq, jt, len;
    long t0;
};

// Workgroups are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8).
// Block b serves unit rank 8*(slot / njt) + b%8 and value tile slot % njt with
// slot = b / 8, so the value tiles of one unit share an XCD (and its L2) and
// are dispatched next to each other.  Unit rank r is head r % H of the
// (r / H)-th sequence in the order given by p.order (identity if NULL).
__device__ __forceinline__ WorkItem decode_work(const KParams& p) {
    WorkItem wi;
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int slot = bid >> 3;
    wi.jt = slot % p.njt_all;
    const int urank = (slot / p.njt_all) * 8 + xcd;
    wi.valid = urank < p.units;
    if (!wi.valid) return wi;
    wi.h = urank % p.H;
    const int srank = urank / p.H;
    wi.seq = p.order ? p.order[srank] : srank;
    if (p.cu_seqlens) {
        wi.t0 = p.cu_seqlens[wi.seq];
        wi.len = p.cu_seqlens[wi.seq + 1] - (int)wi.t0;
    } else {
        wi.t0 = (long)wi.seq * p.T;
        wi.len = p.t_len >= 0 ? p.t_len : p.T;
    }
    return wi;
}

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Raw buffer descriptor over [base, base + bytes).  Loads past the range
// return zero and stores past it are dropped, so a chunk's tail rows need no
// branch: a store that is issued on every path lets the compiler count the
// memory operations in flight exactly (stores and loads share one counter),
// where a store under a branch makes every later wait assume the shorter
// path and so also wait for stores and loads that were issued after the one
// it needs.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    // stride 0, num_records = bytes, dword 3 = 32-bit data format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
// cache policy of a store that is read only much later (non-temporal)
constexpr int CPOL_NT = 2;

// Store N consecutive operand elements to LDS with the widest aligned writes.
template <typename Top, int N>
__device__ __forceinline__ void store_run(Top* p, const Top* v) {
    if constexpr (sizeof(Top) * N >= 16) {
#pragma unroll
        for (int i = 0; i < N * (int)sizeof(Top) / 16; ++i) {
            uint4 u;
            __builtin_memcpy(&u, v + i * (16 / sizeof(Top)), 16);
            reinterpret_cast<uint4*>(p)[i] = u;
        }
    } else if constexpr (sizeof(Top) * N == 8) {
        uint2 u;
        __builtin_memcpy(&u, v, 8);
        *reinterpret_cast<uint2*>(p) = u;
    } else if constexpr (sizeof(Top) * N == 4) {
        uint32_t u;
        __builtin_memcpy(&u, v, 4);
        *reinterpret_cast<uint32_t*>(p) = u;
    } else {
        *p = v[0];
    }
}


// the pipelined bf16 chunk kernel (chunk_fwd_bf16.hip)
hipError_t launch_chunk_bf16(const KParams& p, int dk, int dvt, hipStream_t stream);
bool chunk_bf16_supports(int dvt);

}  // namespace kda
