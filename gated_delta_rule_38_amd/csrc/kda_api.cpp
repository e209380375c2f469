// kda_api.cpp -- the C ABI of libkda: host-side validation, then dispatch to
// the HIP launchers.  Every check runs before any HIP call, so a rejected call
// enqueues nothing and leaves every output untouched.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <new>

#include "../../include/kda.h"
#include "kda_launch.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int kChunk = 64;

bool supported_dim(int d) { return d == 64 || d == 128; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
    bool empty() const { return hi <= lo; }
};

Range range_of(const void* p, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, p ? lo + bytes : lo};
}

bool overlap(Range a, Range b) {
    if (a.empty() || b.empty()) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// n * m with overflow detection
bool mul_ok(size_t a, size_t b, size_t* out) {
    if (a != 0 && b > SIZE_MAX / a) return false;
    *out = a * b;
    return true;
}

bool bytes_of(size_t elems_a, size_t elems_b, size_t elems_c, size_t elems_d, size_t esize,
              size_t* out) {
    size_t x;
    return mul_ok(elems_a, elems_b, &x) && mul_ok(x, elems_c, &x) && mul_ok(x, elems_d, &x) &&
           mul_ok(x, esize, out);
}

float default_scale(float scale, int dk) {
    if (scale > 0.f && isfinite(scale)) return scale;
    return 1.0f / sqrtf((float)dk);
}

bool valid_gate(int gate) {
    return gate == KDA_GATE_CHANNEL || gate == KDA_GATE_HEAD || gate == KDA_GATE_NONE;
}

constexpr unsigned kAllFuse = KDA_FUSE_GATE_LOGITS | KDA_FUSE_BETA_LOGITS | KDA_FUSE_QK_L2NORM;

// flags that the gate kind admits
bool valid_flags(int gate, unsigned flags) {
    if (flags & ~kAllFuse) return false;
    return !(gate == KDA_GATE_NONE && (flags & KDA_FUSE_GATE_LOGITS));
}

// alpha values per token and head for a gate
size_t gate_width(int gate, int dk) {
    return gate == KDA_GATE_CHANNEL ? (size_t)dk : gate == KDA_GATE_HEAD ? 1 : 0;
}

bool env_generic() {
    const char* s = getenv("KDA_CHUNK_GENERIC");
    return s && s[0] == '1';
}

int env_dvt() {
    const char* s = getenv("KDA_CHUNK_DVT");
    if (!s) return 0;
    int v = atoi(s);
    return (v == 16 || v == 32 || v == 64) ? v : 0;
}

kda_status chunk_fwd_impl(const void* q, const void* k, const void* v, const void* alpha,
                          const float* beta, const float* initial_state, void* o,
                          float* final_state, int B, int T, int H, int dk, int dv,
                          kda_dtype dtype, int gate, unsigned flags, const int* cu_seqlens_dev,
                          const int* cu_seqlens_host, int num_seqs, float scale,
                          int chunk_size, void* workspace, size_t workspace_bytes,
                          hipStream_t stream, bool noalloc = false);
kda_status recurrent_step_impl(const void* q, const void* k, const void* v, const void* alpha,
                               const float* beta, float* state, void* o, int N, int H, int dk,
                               int dv, kda_dtype dtype, int gate, unsigned flags, float scale,
                               hipStream_t stream);

}  // namespace

extern "C" {

int kda_version(void) { return kVersion; }

const char* kda_status_string(kda_status status) {
    switch (status) {
        case KDA_SUCCESS: return "KDA_SUCCESS";
        case KDA_ERROR_INVALID_VALUE: return "KDA_ERROR_INVALID_VALUE";
        case KDA_ERROR_NOT_SUPPORTED: return "KDA_ERROR_NOT_SUPPORTED";
        case KDA_ERROR_MISALIGNED: return "KDA_ERROR_MISALIGNED";
        case KDA_ERROR_INSUFFICIENT_WORKSPACE: return "KDA_ERROR_INSUFFICIENT_WORKSPACE";
        case KDA_ERROR_HIP: return "KDA_ERROR_HIP";
    }
    return "unknown status";
}

size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int num_seqs,
                                    kda_dtype dtype) {
    if (B < 0 || T < 0 || H < 0 || num_seqs < 0) return 0;
    if (!supported_dim(dk) || !supported_dim(dv)) return 0;
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return 0;
    if (num_seqs == 0) return 0;
    return ((size_t)num_seqs * 4 + 255) / 256 * 256;
}

size_t kda_chunk_fwd_split_workspace_size(int B, int T, int H, int dk, int dv,
                                          kda_dtype dtype) {
    if (B < 0 || T < 0 || H < 0 || dtype != KDA_DTYPE_BF16) return 0;
    return kda::chunk_split_plan(B, T, H, dk, dv).bytes;
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, const float* initial_state, void* o,
                         float* final_state, int B, int T, int H, int dk, int dv,
                         kda_dtype dtype, const int* cu_seqlens_dev,
                         const int* cu_seqlens_host, int num_seqs, float scale,
                         int chunk_size, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, alpha, beta, initial_state, o, final_state, B, T, H, dk, dv,
                          dtype, KDA_GATE_CHANNEL, 0u, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                          scale, chunk_size, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, const float* initial_state, void* o,
                               float* final_state, int B, int T, int H, int dk, int dv,
                               kda_dtype dtype, kda_gate gate, const int* cu_seqlens_dev,
                               const int* cu_seqlens_host, int num_seqs, float scale,
                               int chunk_size, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, alpha, beta, initial_state, o, final_state, B, T, H, dk, dv,
                          dtype, (int)gate, 0u, cu_seqlens_dev, cu_seqlens_host, num_seqs, scale,
                          chunk_size, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_fused(const void* q, const void* k, const void* v, const void* gate,
                               const float* beta, const float* initial_state, void* o,
                               float* final_state, int B, int T, int H, int dk, int dv,
                               kda_dtype dtype, kda_gate gate_kind, unsigned flags,
                               const int* cu_seqlens_dev, const int* cu_seqlens_host,
                               int num_seqs, float scale, int chunk_size, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, gate, beta, initial_state, o, final_state, B, T, H, dk, dv,
                          dtype, (int)gate_kind, flags, cu_seqlens_dev, cu_seqlens_host,
                          num_seqs, scale, chunk_size, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta,
                                 const float* initial_state, void* o, float* final_state, int B,
                                 int T, int H, int dk, int dv, kda_dtype dtype,
                                 const int* cu_seqlens_dev, const int* cu_seqlens_host,
                                 int num_seqs, float scale, int chunk_size, hipStream_t stream) {
    static_assert(KDA_NOALLOC_MAX_SEQS == kda::NOALLOC_MAX_SEQS, "scratch size");
    return chunk_fwd_impl(q, k, v, alpha, beta, initial_state, o, final_state, B, T, H, dk, dv,
                          dtype, KDA_GATE_CHANNEL, 0u, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                          scale, chunk_size, nullptr, 0, stream, true);
}

kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, float* state, void* o, int N, int H, int dk,
                              int dv, kda_dtype dtype, float scale, hipStream_t stream) {
    return recurrent_step_impl(q, k, v, alpha, beta, state, o, N, H, dk, dv, dtype,
                               KDA_GATE_CHANNEL, 0u, scale, stream);
}

kda_status kda_recurrent_step_gated(const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta, float* state,
                                    void* o, int N, int H, int dk, int dv, kda_dtype dtype,
                                    kda_gate gate, float scale, hipStream_t stream) {
    return recurrent_step_impl(q, k, v, alpha, beta, state, o, N, H, dk, dv, dtype, (int)gate,
                               0u, scale, stream);
}

kda_status kda_recurrent_step_fused(const void* q, const void* k, const void* v,
                                    const void* gate, const float* beta, float* state, void* o,
                                    int N, int H, int dk, int dv, kda_dtype dtype,
                                    kda_gate gate_kind, unsigned flags, float scale,
                                    hipStream_t stream) {
    return recurrent_step_impl(q, k, v, gate, beta, state, o, N, H, dk, dv, dtype,
                               (int)gate_kind, flags, scale, stream);
}

size_t kda_backward_workspace_size(int B, int T, int H, int dk, int dv, int num_seqs,
                                   kda_dtype dtype) {
    if (B < 0 || T < 0 || H < 0 || num_seqs < 0) return 0;
    if (!supported_dim(dk) || !supported_dim(dv)) return 0;
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return 0;
    const long tokens = num_seqs > 0 ? (long)T : (long)B * T;
    const int nseq = num_seqs > 0 ? num_seqs : B;
    if (nseq == 0 || H == 0) return 0;
    return dtype == KDA_DTYPE_BF16 ? kda::bwd_chunk_workspace_bytes(tokens, nseq, H, dk, dv)
                                   : kda::backward_workspace_bytes(tokens, nseq, H, dk, dv);
}

kda_status kda_backward(const void* q, const void* k, const void* v, const float* alpha,
                        const float* beta, const float* initial_state, const void* dout,
                        const float* dfinal_state, float* dq, float* dk, float* dv,
                        float* dalpha, float* dbeta, float* dinitial_state, int B, int T, int H,
                        int dk_dim, int dv_dim, kda_dtype dtype, const int* cu_seqlens_dev,
                        const int* cu_seqlens_host, int num_seqs, float scale, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    try {
        if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERROR_INVALID_VALUE;
        if (B < 0 || T < 0 || H < 0 || num_seqs < 0) return KDA_ERROR_INVALID_VALUE;
        if (!supported_dim(dk_dim) || !supported_dim(dv_dim)) return KDA_ERROR_NOT_SUPPORTED;
        const bool varlen = num_seqs > 0;
        if (!varlen && (cu_seqlens_dev || cu_seqlens_host)) return KDA_ERROR_INVALID_VALUE;
        int nstates = B;
        if (varlen) {
            if (!cu_seqlens_dev || !cu_seqlens_host || B != 1) return KDA_ERROR_INVALID_VALUE;
            if (cu_seqlens_host[0] != 0 || cu_seqlens_host[num_seqs] != T)
                return KDA_ERROR_INVALID_VALUE;
            for (int n = 0; n < num_seqs; ++n)
                if (cu_seqlens_host[n + 1] < cu_seqlens_host[n]) return KDA_ERROR_INVALID_VALUE;
            if ((reinterpret_cast<uintptr_t>(cu_seqlens_dev) & 3u) != 0)
                return KDA_ERROR_MISALIGNED;
            nstates = num_seqs;
        }
        const size_t es = dtype == KDA_DTYPE_BF16 ? 2 : 4;
        size_t b_qk, b_v, b_qk4, b_v4, b_b, b_s;
        if (!bytes_of(B, T, H, dk_dim, es, &b_qk) || !bytes_of(B, T, H, dv_dim, es, &b_v) ||
            !bytes_of(B, T, H, dk_dim, 4, &b_qk4) || !bytes_of(B, T, H, dv_dim, 4, &b_v4) ||
            !bytes_of(B, T, H, 1, 4, &b_b) || !bytes_of(nstates, H, dk_dim, dv_dim, 4, &b_s))
            return KDA_ERROR_INVALID_VALUE;
        if ((long long)nstates * H > (1LL << 30)) return KDA_ERROR_NOT_SUPPORTED;
        if ((long long)B * T > (1LL << 31) - 1) return KDA_ERROR_NOT_SUPPORTED;
        const size_t tokens = (size_t)B * T * H;
        const size_t units = (size_t)nstates * H;
        if (tokens > 0 && (!q || !k || !v || !alpha || !beta || !dout || !dq || !dk || !dv ||
                           !dalpha || !dbeta))
            return KDA_ERROR_INVALID_VALUE;
        if (units > 0 && !dinitial_state) return KDA_ERROR_INVALID_VALUE;
        const void* elems[] = {q, k};
        for (const void* ptr : elems)
            if (!aligned(ptr, es)) return KDA_ERROR_MISALIGNED;
        // the chunk form (bf16) reads q, k and alpha in pairs of channels
        if (dtype == KDA_DTYPE_BF16 && (!aligned(q, 8) || !aligned(k, 8) || !aligned(alpha, 8)))
            return KDA_ERROR_MISALIGNED;
        // v and dout are read as runs of four elements
        if (!aligned(v, 4 * es) || !aligned(dout, 4 * es)) return KDA_ERROR_MISALIGNED;
        const void* words[] = {alpha, beta, dq, dk, dv, dalpha, dbeta};
        for (const void* ptr : words)
            if (!aligned(ptr, 4)) return KDA_ERROR_MISALIGNED;
        const void* quads[] = {initial_state, dfinal_state, dinitial_state};
        for (const void* ptr : quads)
            if (!aligned(ptr, 16)) return KDA_ERROR_MISALIGNED;
        if (!aligned(workspace, 256)) return KDA_ERROR_MISALIGNED;
        const size_t need_ws =
            kda_backward_workspace_size(B, T, H, dk_dim, dv_dim, num_seqs, dtype);
        if (need_ws > 0 && (!workspace || workspace_bytes < need_ws))
            return KDA_ERROR_INSUFFICIENT_WORKSPACE;
        // outputs against inputs and against each other
        const Range outs[] = {range_of(dq, tokens ? b_qk4 : 0), range_of(dk, tokens ? b_qk4 : 0),
                              range_of(dv, tokens ? b_v4 : 0), range_of(dalpha, tokens ? b_qk4 : 0),
                              range_of(dbeta, tokens ? b_b : 0),
                              range_of(dinitial_state, units ? b_s : 0),
                              range_of(workspace, need_ws)};
        const Range ins[] = {range_of(q, b_qk), range_of(k, b_qk), range_of(v, b_v),
                             range_of(alpha, b_qk4), range_of(beta, b_b), range_of(dout, b_v),
                             range_of(initial_state, units ? b_s : 0),
                             range_of(dfinal_state, units ? b_s : 0),
                             range_of(cu_seqlens_dev, varlen ? (size_t)(num_seqs + 1) * 4 : 0)};
        for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
            for (const Range& r : ins)
                if (overlap(outs[i], r)) return KDA_ERROR_INVALID_VALUE;
            for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
                if (overlap(outs[i], outs[j])) return KDA_ERROR_INVALID_VALUE;
        }
        if (units == 0) return KDA_SUCCESS;

        kda::BwdArgs a;
        a.q = q; a.k = k; a.v = v; a.dout = dout;
        a.alpha = alpha; a.beta = beta; a.s0 = initial_state; a.dsT = dfinal_state;
        a.g_q = dq; a.g_k = dk; a.g_v = dv; a.g_alpha = dalpha; a.g_beta = dbeta;
        a.g_s0 = dinitial_state;
        a.B = B; a.T = T; a.H = H; a.dk = dk_dim; a.dv = dv_dim;
        a.bf16 = dtype == KDA_DTYPE_BF16;
        a.cu_seqlens = varlen ? cu_seqlens_dev : nullptr;
        a.num_seqs = varlen ? num_seqs : 0;
        a.scale = default_scale(scale, dk_dim);
        a.workspace = workspace;
        const hipError_t e = a.bf16 ? kda::launch_bwd_chunk(a, stream)
                                    : kda::launch_backward(a, stream);
        return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_HIP;
    } catch (...) {
        return KDA_ERROR_HIP;
    }
}

}  // extern "C"

namespace {

kda_status chunk_fwd_impl(const void* q, const void* k, const void* v, const void* alpha,
                          const float* beta, const float* initial_state, void* o,
                          float* final_state, int B, int T, int H, int dk, int dv,
                          kda_dtype dtype, int gate, unsigned flags, const int* cu_seqlens_dev,
                          const int* cu_seqlens_host, int num_seqs, float scale,
                          int chunk_size, void* workspace, size_t workspace_bytes,
                          hipStream_t stream, bool noalloc) {
    try {
        if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERROR_INVALID_VALUE;
        if (!valid_gate(gate) || !valid_flags(gate, flags)) return KDA_ERROR_INVALID_VALUE;
        if (gate == KDA_GATE_NONE && alpha) return KDA_ERROR_INVALID_VALUE;
        // the no-allocation variant keeps the sequence order in a fixed device array
        if (noalloc && num_seqs > KDA_NOALLOC_MAX_SEQS) return KDA_ERROR_NOT_SUPPORTED;
        if (B < 0 || T < 0 || H < 0 || num_seqs < 0) return KDA_ERROR_INVALID_VALUE;
        if (chunk_size != kChunk) return KDA_ERROR_NOT_SUPPORTED;
        if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERROR_NOT_SUPPORTED;
        const bool varlen = num_seqs > 0;
        if (!varlen && (cu_seqlens_dev || cu_seqlens_host)) return KDA_ERROR_INVALID_VALUE;
        const size_t es = dtype == KDA_DTYPE_BF16 ? 2 : 4;
        const size_t ges = (flags & KDA_FUSE_GATE_LOGITS) ? es : 4;  // gate element size
        int nstates = B;
        if (varlen) {
            if (!cu_seqlens_dev || !cu_seqlens_host || B != 1) return KDA_ERROR_INVALID_VALUE;
            if (cu_seqlens_host[0] != 0 || cu_seqlens_host[num_seqs] != T)
                return KDA_ERROR_INVALID_VALUE;
            for (int n = 0; n < num_seqs; ++n)
                if (cu_seqlens_host[n + 1] < cu_seqlens_host[n]) return KDA_ERROR_INVALID_VALUE;
            if ((reinterpret_cast<uintptr_t>(cu_seqlens_dev) & 3u) != 0)
                return KDA_ERROR_MISALIGNED;
            nstates = num_seqs;
        }
        size_t b_qk, b_v, b_a, b_b, b_s;
        if (!bytes_of(B, T, H, dk, es, &b_qk) || !bytes_of(B, T, H, dv, es, &b_v) ||
            !bytes_of(B, T, H, gate_width(gate, dk), ges, &b_a) || !bytes_of(B, T, H, 1, 4, &b_b) ||
            !bytes_of(nstates, H, dk, dv, 4, &b_s))
            return KDA_ERROR_INVALID_VALUE;
        // grid and index limits of the kernels
        if ((long long)nstates * H * (dv / 16) > (1LL << 30)) return KDA_ERROR_NOT_SUPPORTED;
        if ((long long)B * T > (1LL << 31) - 1) return KDA_ERROR_NOT_SUPPORTED;

        const size_t tokens = (size_t)B * T * H;
        const size_t units = (size_t)nstates * H;
        if (tokens > 0 && (!q || !k || !v || !beta || !o || (gate != KDA_GATE_NONE && !alpha)))
            return KDA_ERROR_INVALID_VALUE;
        // q, k and a per-channel alpha are read in pairs; the rest element by element
        const void* pairs[] = {q, k, gate == KDA_GATE_CHANNEL ? alpha : nullptr};
        for (const void* ptr : pairs)
            if (!aligned(ptr, 8)) return KDA_ERROR_MISALIGNED;
        if (!aligned(alpha, ges)) return KDA_ERROR_MISALIGNED;
        if (!aligned(v, es) || !aligned(o, es)) return KDA_ERROR_MISALIGNED;
        const void* words[] = {beta, initial_state, final_state, workspace};
        for (const void* ptr : words)
            if (!aligned(ptr, 4)) return KDA_ERROR_MISALIGNED;

        const size_t min_ws =
            noalloc ? 0 : kda_chunk_fwd_workspace_size(B, T, H, dk, dv, num_seqs, dtype);
        if (min_ws > 0 && (!workspace || workspace_bytes < min_ws))
            return KDA_ERROR_INSUFFICIENT_WORKSPACE;
        // Dense bf16 calls whose workspace holds the two-segment path's
        // buffers (256-byte aligned) take that path when o allows its 8-byte
        // accesses; overrides of the kernel choice keep the single pass.
        const size_t split_ws = (noalloc || varlen || env_generic() || env_dvt())
                                    ? 0 : kda_chunk_fwd_split_workspace_size(B, T, H, dk, dv, dtype);
        const bool split = split_ws > 0 && workspace && workspace_bytes >= split_ws &&
                           aligned(workspace, 256) && aligned(o, 8);
        const size_t need_ws = split ? split_ws : min_ws;

        // outputs must not overlap inputs, each other or the workspace; the one
        // allowed alias is an in-place state (final_state == initial_state)
        const Range r_o = range_of(o, tokens ? b_v : 0);
        const Range r_f = range_of(final_state, units ? b_s : 0);
        const Range r_ws = range_of(workspace, need_ws);
        const Range ins[] = {range_of(q, b_qk), range_of(k, b_qk), range_of(v, b_v),
                             range_of(alpha, b_a), range_of(beta, b_b),
                             range_of(cu_seqlens_dev, varlen ? (size_t)(num_seqs + 1) * 4 : 0)};
        for (const Range& r : ins) {
            if (overlap(r_o, r) || overlap(r_f, r) || overlap(r_ws, r))
                return KDA_ERROR_INVALID_VALUE;
        }
        const Range r_i = range_of(initial_state, units ? b_s : 0);
        if (overlap(r_o, r_i) || overlap(r_o, r_f) || overlap(r_o, r_ws) || overlap(r_f, r_ws) ||
            overlap(r_i, r_ws))
            return KDA_ERROR_INVALID_VALUE;
        if (overlap(r_f, r_i) && final_state != initial_state) return KDA_ERROR_INVALID_VALUE;

        if (units == 0) return KDA_SUCCESS;

        kda::ChunkArgs a;
        a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
        a.s0 = initial_state; a.o = o; a.sT = final_state;
        a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv;
        a.bf16 = dtype == KDA_DTYPE_BF16;
        a.gate = gate;
        a.fuse = (int)flags;
        a.cu_seqlens = varlen ? cu_seqlens_dev : nullptr;
        a.num_seqs = varlen ? num_seqs : 0;
        a.order = (varlen && num_seqs <= 65536) ? static_cast<int*>(workspace) : nullptr;
        a.split_ws = split ? workspace : nullptr;
        if (noalloc && varlen) {
            int* order = nullptr;
            if (kda::noalloc_order_buffer(stream, &order) != hipSuccess) return KDA_ERROR_HIP;
            a.order = order;
        }
        a.scale = default_scale(scale, dk);
        a.dvt = env_dvt();
        a.generic = env_generic();
        return kda::launch_chunk_fwd(a, stream) == hipSuccess ? KDA_SUCCESS : KDA_ERROR_HIP;
    } catch (...) {
        return KDA_ERROR_HIP;
    }
}

kda_status recurrent_step_impl(const void* q, const void* k, const void* v, const void* alpha,
                               const float* beta, float* state, void* o, int N, int H, int dk,
                               int dv, kda_dtype dtype, int gate, unsigned flags, float scale,
                               hipStream_t stream) {
    try {
        if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERROR_INVALID_VALUE;
        if (!valid_gate(gate) || !valid_flags(gate, flags)) return KDA_ERROR_INVALID_VALUE;
        if (gate == KDA_GATE_NONE && alpha) return KDA_ERROR_INVALID_VALUE;
        if (N < 0 || H < 0) return KDA_ERROR_INVALID_VALUE;
        if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERROR_NOT_SUPPORTED;
        if ((long long)N * H > (1LL << 31) - 1) return KDA_ERROR_NOT_SUPPORTED;
        const size_t units = (size_t)N * H;
        if (units == 0) return KDA_SUCCESS;
        if (!q || !k || !v || !beta || !state || !o || (gate != KDA_GATE_NONE && !alpha))
            return KDA_ERROR_INVALID_VALUE;
        const size_t es = dtype == KDA_DTYPE_BF16 ? 2 : 4;
        // the state is streamed as float4; everything else element by element
        if (!aligned(state, 16)) return KDA_ERROR_MISALIGNED;
        const size_t ges = (flags & KDA_FUSE_GATE_LOGITS) ? es : 4;  // gate element size
        if (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(o, es) ||
            !aligned(alpha, ges) || !aligned(beta, 4))
            return KDA_ERROR_MISALIGNED;
        const Range r_s = range_of(state, units * dk * dv * 4);
        const Range r_o = range_of(o, units * dv * es);
        const Range ins[] = {range_of(q, units * dk * es), range_of(k, units * dk * es),
                             range_of(v, units * dv * es),
                             range_of(alpha, units * gate_width(gate, dk) * ges),
                             range_of(beta, units * 4)};
        for (const Range& r : ins)
            if (overlap(r_s, r) || overlap(r_o, r)) return KDA_ERROR_INVALID_VALUE;
        if (overlap(r_s, r_o)) return KDA_ERROR_INVALID_VALUE;

        kda::StepArgs a;
        a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.state = state; a.o = o;
        a.N = N; a.H = H; a.dk = dk; a.dv = dv;
        a.bf16 = dtype == KDA_DTYPE_BF16;
        a.gate = gate;
        a.fuse = (int)flags;
        a.scale = default_scale(scale, dk);
        return kda::launch_recurrent_step(a, stream) == hipSuccess ? KDA_SUCCESS : KDA_ERROR_HIP;
    } catch (...) {
        return KDA_ERROR_HIP;
    }
}

}  // namespace

extern "C" {

kda_status kda_gdn2_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                              const float* erase, const float* write,
                              const float* initial_state, void* o, float* final_state, int B,
                              int T, int H, int dk, int dv, kda_dtype dtype,
                              const int* cu_seqlens_dev, const int* cu_seqlens_host,
                              int num_seqs, float scale, int chunk_size, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    try {
        if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERROR_INVALID_VALUE;
        if (B < 0 || T < 0 || H < 0 || num_seqs < 0) return KDA_ERROR_INVALID_VALUE;
        if (chunk_size != kChunk) return KDA_ERROR_NOT_SUPPORTED;
        if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERROR_NOT_SUPPORTED;
        // the chunk kernel keeps bf16 operands only (float32 ones do not fit in LDS)
        if (dtype != KDA_DTYPE_BF16) return KDA_ERROR_NOT_SUPPORTED;
        const bool varlen = num_seqs > 0;
        if (!varlen && (cu_seqlens_dev || cu_seqlens_host)) return KDA_ERROR_INVALID_VALUE;
        const size_t es = 2;
        int nstates = B;
        if (varlen) {
            if (!cu_seqlens_dev || !cu_seqlens_host || B != 1) return KDA_ERROR_INVALID_VALUE;
            if (cu_seqlens_host[0] != 0 || cu_seqlens_host[num_seqs] != T)
                return KDA_ERROR_INVALID_VALUE;
            for (int n = 0; n < num_seqs; ++n)
                if (cu_seqlens_host[n + 1] < cu_seqlens_host[n]) return KDA_ERROR_INVALID_VALUE;
            if ((reinterpret_cast<uintptr_t>(cu_seqlens_dev) & 3u) != 0)
                return KDA_ERROR_MISALIGNED;
            nstates = num_seqs;
        }
        size_t b_qk, b_v, b_g, b_s;
        if (!bytes_of(B, T, H, dk, es, &b_qk) || !bytes_of(B, T, H, dv, es, &b_v) ||
            !bytes_of(B, T, H, dk, 4, &b_g) || !bytes_of(nstates, H, dk, dv, 4, &b_s))
            return KDA_ERROR_INVALID_VALUE;
        if ((long long)nstates * H * (dv / 16) > (1LL << 30)) return KDA_ERROR_NOT_SUPPORTED;
        if ((long long)B * T > (1LL << 31) - 1) return KDA_ERROR_NOT_SUPPORTED;
        const size_t tokens = (size_t)B * T * H;
        const size_t units = (size_t)nstates * H;
        if (tokens > 0 && (!q || !k || !v || !erase || !write || !o))
            return KDA_ERROR_INVALID_VALUE;
        // q, k and the three gates are read in pairs of channels
        const void* pairs[] = {q, k, alpha, erase, write};
        for (const void* ptr : pairs)
            if (!aligned(ptr, 8)) return KDA_ERROR_MISALIGNED;
        if (!aligned(v, es) || !aligned(o, es)) return KDA_ERROR_MISALIGNED;
        const void* words[] = {initial_state, final_state, workspace};
        for (const void* ptr : words)
            if (!aligned(ptr, 4)) return KDA_ERROR_MISALIGNED;
        const size_t need_ws = kda_chunk_fwd_workspace_size(B, T, H, dk, dv, num_seqs, dtype);
        if (need_ws > 0 && (!workspace || workspace_bytes < need_ws))
            return KDA_ERROR_INSUFFICIENT_WORKSPACE;
        const Range r_o = range_of(o, tokens ? b_v : 0);
        const Range r_f = range_of(final_state, units ? b_s : 0);
        const Range r_ws = range_of(workspace, need_ws);
        const Range ins[] = {range_of(q, b_qk), range_of(k, b_qk), range_of(v, b_v),
                             range_of(alpha, tokens ? b_g : 0), range_of(erase, b_g),
                             range_of(write, b_g),
                             range_of(cu_seqlens_dev, varlen ? (size_t)(num_seqs + 1) * 4 : 0)};
        for (const Range& r : ins)
            if (overlap(r_o, r) || overlap(r_f, r) || overlap(r_ws, r))
                return KDA_ERROR_INVALID_VALUE;
        const Range r_i = range_of(initial_state, units ? b_s : 0);
        if (overlap(r_o, r_i) || overlap(r_o, r_f) || overlap(r_o, r_ws) || overlap(r_f, r_ws) ||
            overlap(r_i, r_ws))
            return KDA_ERROR_INVALID_VALUE;
        if (overlap(r_f, r_i) && final_state != initial_state) return KDA_ERROR_INVALID_VALUE;
        if (units == 0) return KDA_SUCCESS;

        kda::Gdn2ChunkArgs a;
        a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.erase = erase; a.write = write;
        a.s0 = initial_state; a.o = o; a.sT = final_state;
        a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv;
        a.bf16 = true;
        a.cu_seqlens = varlen ? cu_seqlens_dev : nullptr;
        a.num_seqs = varlen ? num_seqs : 0;
        a.order = (varlen && num_seqs <= 65536) ? static_cast<int*>(workspace) : nullptr;
        a.scale = default_scale(scale, dk);
        a.dvt = env_dvt();
        return kda::launch_gdn2_chunk_fwd(a, stream) == hipSuccess ? KDA_SUCCESS : KDA_ERROR_HIP;
    } catch (...) {
        return KDA_ERROR_HIP;
    }
}

kda_status kda_gdn2_recurrent_step(const void* q, const void* k, const void* v,
                                   const float* alpha, const float* erase, const float* write,
                                   float* state, void* o, int N, int H, int dk, int dv,
                                   kda_dtype dtype, float scale, hipStream_t stream) {
    try {
        if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERROR_INVALID_VALUE;
        if (N < 0 || H < 0) return KDA_ERROR_INVALID_VALUE;
        if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERROR_NOT_SUPPORTED;
        if ((long long)N * H > (1LL << 31) - 1) return KDA_ERROR_NOT_SUPPORTED;
        const size_t units = (size_t)N * H;
        if (units == 0) return KDA_SUCCESS;
        if (!q || !k || !v || !erase || !write || !state || !o) return KDA_ERROR_INVALID_VALUE;
        const size_t es = dtype == KDA_DTYPE_BF16 ? 2 : 4;
        if (!aligned(state, 16)) return KDA_ERROR_MISALIGNED;
        if (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(o, es) ||
            !aligned(alpha, 4) || !aligned(erase, 4) || !aligned(write, 4))
            return KDA_ERROR_MISALIGNED;
        const Range r_s = range_of(state, units * dk * dv * 4);
        const Range r_o = range_of(o, units * dv * es);
        const Range ins[] = {range_of(q, units * dk * es), range_of(k, units * dk * es),
                             range_of(v, units * dv * es), range_of(alpha, units * dk * 4),
                             range_of(erase, units * dk * 4), range_of(write, units * dk * 4)};
        for (const Range& r : ins)
            if (overlap(r_s, r) || overlap(r_o, r)) return KDA_ERROR_INVALID_VALUE;
        if (overlap(r_s, r_o)) return KDA_ERROR_INVALID_VALUE;
        kda::Gdn2StepArgs a;
        a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.erase = erase; a.write = write;
        a.state = state; a.o = o;
        a.N = N; a.H = H; a.dk = dk; a.dv = dv;
        a.bf16 = dtype == KDA_DTYPE_BF16;
        a.scale = default_scale(scale, dk);
        return kda::launch_gdn2_step(a, stream) == hipSuccess ? KDA_SUCCESS : KDA_ERROR_HIP;
    } catch (...) {
        return KDA_ERROR_HIP;
    }
}

}  // extern "C"
