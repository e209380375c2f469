// chunk_walk.h -- the exact token-by-token walk that the chunk-wise forward
// kernels fall back to for a work item whose decays leave the range of the
// chunk form.
//
// The chunk form scales each key and query row of a chunk by P_r / Pm and
// Pm / P_r, with P_r the product of alpha over the chunk's tokens 0..r and
// Pm = P_31 (the reference in the middle of the chunk).  Every such factor lies
// between the smaller of the two half-chunk products, P_31 and P_63 / P_31, and
// its inverse; while both are at least DECAY_FLOOR = 2^-100 in every key
// channel the scaled operands stay in fp32's (and bf16's) normal range with
// 26 bits to spare for the magnitudes of k and q themselves.  The pages allow
// any alpha in (0, 1] ("Kimi Delta Attention", section "一、Diag(α_t)：通道级
// 遗忘"), so a chunk below the floor is flagged instead, and the work item
// (one unit's slice of value columns) is recomputed at the end of the same
// launch by token_walk: the update of "KDA 的更新式" (or its Gated DeltaNet-2
// form) one token at a time, which involves no ratio of decays and is exact
// for any alpha.  In-domain work items never enter it.
#pragma once

#include "chunk_common.h"

namespace kda {

constexpr float DECAY_FLOOR = 0x1p-100f;

// Whether a chunk with half-chunk decay products first = P_31 and
// second = P_63 / P_31 (one key channel) leaves the chunk form's range.  A NaN
// decay is not flagged: it propagates through the chunk form as it would here.
__device__ __forceinline__ bool decay_out_of_range(float first, float second) {
    return first < DECAY_FLOOR || second < DECAY_FLOOR;
}

struct WalkArgs {
    const void *q, *k, *v;
    const void *alpha;           // float32 decays, or logits in the dtype of q (FUSE_GATE_LOGITS)
    const float *beta;           // KDA: [token, H] write strengths, or logits (FUSE_BETA_LOGITS)
    const float *erase, *write;  // Gated DeltaNet-2: [token, H, dk]
    const float *s0;
    void *o;
    float *sT;
    float *ckpt;  // chunk-start states in the chunk kernels' slot layout, or NULL
    int H, dv;
    int gate;     // 0 per key channel, 1 per head, 2 none (alpha NULL in Gated DeltaNet-2)
    int fuse;     // FUSE_* bits (KDA only)
    float scale;
    bool ident = false;  // start from the identity (dv == dk) with every value zero
};

template <int DVT, int NTHR, bool GDN2>
struct WalkShape {
    static constexpr int NACT = NTHR >= 512 ? 512 : 256;        // threads that take part
    static constexpr int NR = GDN2 ? 4 : 5;                     // quantities summed per column
    static constexpr int NSLOT = DVT < 64 ? NACT / 64 : NACT / DVT;
    static constexpr size_t lds_bytes = (size_t)2 * NSLOT * DVT * NR * 4;
};

// Recompute unit (seq, h) -- tokens t0 .. t0 + len - 1 -- on value columns
// col0 .. col0 + DVT - 1: its outputs (if a.o), its final state (if a.sT) and
// its chunk-start states (if a.ckpt), from a.s0.  All NTHR threads of the
// workgroup call it (it synchronises them); thread (rg, c) of the first NACT
// holds rows rg*RPT .. rg*RPT + RPT - 1 of column c of the state slice.  Per
// token, with alpha, k and q of the token:
//   S~ = Diag(alpha) S,  vh = S~^T k,  p = S~^T q
//   KDA:       u = beta (v - vh),  S = S~ + k u^T,  o = scale (p + (k.q) u)
//   DeltaNet-2: S = S~ - (e k) vh^T + (w k) v^T,    o = scale (p - ((e k).q) vh + ((w k).q) v)
// (with FUSE_QK_L2NORM, k and q are first divided by their norms; every sum
// over the key channels is formed once per token).  With a.ident the walk
// starts from the identity instead of a.s0 and reads every value as zero.
// lds: lds_bytes of WalkShape, free for the walk.
template <typename Tin, int DK, int DVT, int NTHR, bool GDN2>
__device__ __forceinline__ void token_walk(const WalkArgs& a, int seq, int h, long t0, int len,
                                           int col0, float* lds) {
    using W = WalkShape<DVT, NTHR, GDN2>;
    constexpr int NACT = W::NACT, NR = W::NR, NSLOT = W::NSLOT;
    constexpr int NRG = NACT / DVT;  // row groups
    constexpr int RPT = DK / NRG;    // state rows per thread
    static_assert(DVT <= NACT && RPT >= 1 && RPT * NRG == DK, "walk shape");

    const Tin* __restrict__ gq = static_cast<const Tin*>(a.q);
    const Tin* __restrict__ gk = static_cast<const Tin*>(a.k);
    const Tin* __restrict__ gv = static_cast<const Tin*>(a.v);
    const float* __restrict__ ga = static_cast<const float*>(a.alpha);
    const Tin* __restrict__ gg = static_cast<const Tin*>(a.alpha);
    Tin* __restrict__ go = static_cast<Tin*>(a.o);
    const bool gl = !GDN2 && (a.fuse & FUSE_GATE_LOGITS);
    const bool bl = !GDN2 && (a.fuse & FUSE_BETA_LOGITS);
    const bool qn = !GDN2 && (a.fuse & FUSE_QK_L2NORM);
    const int H = a.H, DV = a.dv;

    const int tid = threadIdx.x;
    const bool act = tid < NACT;
    const int c = tid % DVT, rg = tid / DVT;
    const int r0 = rg * RPT;
    const size_t sbase = ((size_t)seq * H + h) * DK * DV;
    const size_t slot0 = (size_t)(t0 / CH + 2 * (long)seq);

    float S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        S[i] = !act ? 0.f
             : a.ident ? (r0 + i == col0 + c ? 1.f : 0.f)
             : a.s0 ? a.s0[sbase + (size_t)(r0 + i) * DV + col0 + c] : 0.f;
    auto store_state = [&](float* dst) {
        if (!act) return;
#pragma unroll
        for (int i = 0; i < RPT; ++i) dst[(size_t)(r0 + i) * DV + col0 + c] = S[i];
    };

    for (int t = 0; t < len; ++t) {
        if (a.ckpt && t % CH == 0) store_state(a.ckpt + ((slot0 + t / CH) * H + h) * DK * DV);
        const size_t tok = (size_t)(t0 + t) * H + h;
        float part[NR];
#pragma unroll
        for (int j = 0; j < NR; ++j) part[j] = 0.f;
        float kk[RPT], ek[RPT], wk[RPT];
        if (act) {
            float ah = 1.f;  // a decay shared by the token's channels
            if (!GDN2 && a.gate == 1) ah = gl ? sigmoid_f(to_f32(gg[tok])) : ga[tok];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const size_t e = tok * DK + r0 + i;
                float al = ah;
                if (GDN2) al = ga ? ga[e] : 1.f;
                else if (a.gate == 0) al = gl ? sigmoid_f(to_f32(gg[e])) : ga[e];
                kk[i] = to_f32(gk[e]);
                const float qq = to_f32(gq[e]);
                S[i] *= al;
                part[0] += kk[i] * S[i];
                part[1] += qq * S[i];
                if constexpr (GDN2) {
                    ek[i] = a.erase[e] * kk[i];
                    wk[i] = a.write[e] * kk[i];
                    part[2] += ek[i] * qq;
                    part[3] += wk[i] * qq;
                } else {
                    part[2] += kk[i] * qq;
                    part[3] += kk[i] * kk[i];
                    part[4] += qq * qq;
                }
            }
        }
        // sum over the row groups: first those that share a wavefront, then
        // across wavefronts (or row groups, for slices of 64 columns) in LDS,
        // double-buffered by token parity so one barrier per token suffices
        if constexpr (DVT < 64) {
#pragma unroll
            for (int off = DVT; off < 64; off *= 2)
#pragma unroll
                for (int j = 0; j < NR; ++j) part[j] += __shfl_xor(part[j], off, 64);
        }
        float* red = lds + (size_t)(t & 1) * NSLOT * DVT * NR;
        if (act && (DVT >= 64 || (tid & 63) < DVT)) {
            const int slot = DVT < 64 ? tid / 64 : rg;
#pragma unroll
            for (int j = 0; j < NR; ++j) red[(slot * DVT + c) * NR + j] = part[j];
        }
        __syncthreads();
        if (act) {
            float tot[NR];
#pragma unroll
            for (int j = 0; j < NR; ++j) tot[j] = 0.f;
            for (int s = 0; s < NSLOT; ++s)
#pragma unroll
                for (int j = 0; j < NR; ++j) tot[j] += red[(s * DVT + c) * NR + j];
            const float vv = a.ident ? 0.f : to_f32(gv[tok * DV + col0 + c]);
            float ov;
            if constexpr (GDN2) {
                const float vh = tot[0];
                ov = tot[1] - tot[2] * vh + tot[3] * vv;
#pragma unroll
                for (int i = 0; i < RPT; ++i) S[i] += wk[i] * vv - ek[i] * vh;
            } else {
                const float ik = qn ? inv_norm(tot[3]) : 1.f, iq = qn ? inv_norm(tot[4]) : 1.f;
                const float b = bl ? sigmoid_f(a.beta[tok]) : a.beta[tok];
                const float u = b * (vv - tot[0] * ik);
                ov = tot[1] * iq + tot[2] * ik * iq * u;
                const float ku = ik * u;
#pragma unroll
                for (int i = 0; i < RPT; ++i) S[i] += kk[i] * ku;
            }
            if (rg == 0 && go) go[tok * DV + col0 + c] = from_f32<Tin>(a.scale * ov);
        }
    }
    if (a.ckpt) store_state(a.ckpt + ((slot0 + (len + CH - 1) / CH) * H + h) * DK * DV);
    if (a.sT) store_state(a.sT + sbase);
}

}  // namespace kda
