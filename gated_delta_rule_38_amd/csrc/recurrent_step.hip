// recurrent_step.hip -- one-token KDA decode step, state updated in place.
//
// Method: the token-by-token ("fused recurrent") mode of bugfactory.tech news
// 3610, fifth paragraph, applied to a single token: forget per key channel,
// predict with the forgotten state, write beta times the error along the key,
// read with the updated state (same page, second to fourth paragraphs;
// "Kimi Delta Attention", section "KDA 的更新式").
//
// The step is HBM-bound: per (sequence, head) it streams the dk x dv fp32
// state once in and once out (2*dk*dv*4 bytes) against a few hundred bytes of
// token vectors.  One 256-thread workgroup owns one (sequence, head) state:
// thread (rg, cg) holds rows rg*RPG.. of the four value columns 4cg..4cg+3 as
// float4 registers, so every state element is loaded once with 128-bit
// coalesced loads, updated in registers and stored once.  The two reductions
// over the key dimension (vh = S~^T k and p = S~^T q) share one pass; partial
// sums are combined with cross-lane shuffles inside a wavefront and through
// LDS across the four wavefronts.  The read is formed without a second pass
// over the state: o = scale * (S~^T q + e (k . q)) with e = beta (v - vh),
// which equals scale * S_t^T q because S_t = S~ + k e^T.  The new state is
// written with non-temporal stores: nothing reads it again within the step,
// and streaming it past the caches keeps the write-back from competing with
// the reads of the other workgroups (one fifth less time per step, measured).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// QN: q and k are L2-normalised in-kernel (two more reductions, |k|^2 and
// |q|^2, share the pass; every reduced quantity is linear in k or q, so the
// norms are applied to the sums)
template <typename Tin, int DK, int DV, bool QN>
__global__ __launch_bounds__(256) void recurrent_step_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const void* __restrict__ alpha_p, const float* __restrict__ beta, float* __restrict__ state,
    Tin* __restrict__ o, float scale, int gate, int fuse) {
    constexpr int NCG = DV / 4;      // float4 column groups
    constexpr int NRG = 256 / NCG;   // row groups
    constexpr int RPG = DK / NRG;    // rows per thread
    constexpr int NRED = QN ? 11 : 9;  // 4 x vh, 4 x p, k.q (, |k|^2, |q|^2)
    static_assert(NCG <= 64 && 64 % NCG == 0 && RPG >= 1, "shape");

    __shared__ float red[4][NCG][NRED + 1];
    __shared__ float sig[DK];  // sigmoid of per-channel gate logits, formed once per channel

    const int unit = blockIdx.x;  // sequence * H + head
    const int tid = threadIdx.x;
    const int cg = tid % NCG;
    const int rg = tid / NCG;
    const int row0 = rg * RPG;
    float* __restrict__ S = state + (size_t)unit * DK * DV;

    // state first: RPG independent 128-bit loads in flight per thread
    float4 s[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r)
        s[r] = *reinterpret_cast<const float4*>(S + (size_t)(row0 + r) * DV + cg * 4);

    // the forget gate: per key channel, one per (sequence, head), or none;
    // float32 decays, or logits in the dtype of q
    const float* __restrict__ alpha = static_cast<const float*>(alpha_p);
    const Tin* __restrict__ glog = static_cast<const Tin*>(alpha_p);
    const bool gl = fuse & FUSE_GATE_LOGITS;
    float a[RPG], kk[RPG], qq[RPG];
    const float ah = gate == 1 ? (gl ? sigmoid_f(to_f32(glog[unit])) : alpha[unit]) : 1.f;
    if (gate == 0 && gl) {  // every channel's sigmoid once, shared by the NCG column groups
        if (tid < DK) sig[tid] = sigmoid_f(to_f32(glog[(size_t)unit * DK + tid]));
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        const size_t ai = (size_t)unit * DK + row0 + r;
        a[r] = gate == 0 ? (gl ? sig[row0 + r] : alpha[ai]) : ah;
        kk[r] = to_f32(k[(size_t)unit * DK + row0 + r]);
        qq[r] = to_f32(q[(size_t)unit * DK + row0 + r]);
    }
    float vv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vv[j] = to_f32(v[(size_t)unit * DV + cg * 4 + j]);
    const float b = (fuse & FUSE_BETA_LOGITS) ? sigmoid_f(beta[unit]) : beta[unit];

    // forget, then the partial reductions over this thread's rows
    float part[NRED];
#pragma unroll
    for (int i = 0; i < NRED; ++i) part[i] = 0.f;
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        s[r].x *= a[r]; s[r].y *= a[r]; s[r].z *= a[r]; s[r].w *= a[r];
        part[0] += kk[r] * s[r].x; part[1] += kk[r] * s[r].y;
        part[2] += kk[r] * s[r].z; part[3] += kk[r] * s[r].w;
        part[4] += qq[r] * s[r].x; part[5] += qq[r] * s[r].y;
        part[6] += qq[r] * s[r].z; part[7] += qq[r] * s[r].w;
        part[8] += kk[r] * qq[r];
        if constexpr (QN) {
            part[9] += kk[r] * kk[r];
            part[10] += qq[r] * qq[r];
        }
    }
    // across the row groups that share a wavefront
#pragma unroll
    for (int off = NCG; off < 64; off *= 2) {
#pragma unroll
        for (int i = 0; i < NRED; ++i) part[i] += __shfl_xor(part[i], off, 64);
    }
    const int wave = tid / 64;
    if ((tid % 64) < NCG) {
#pragma unroll
        for (int i = 0; i < NRED; ++i) red[wave][cg][i] = part[i];
    }
    __syncthreads();
    float tot[NRED];
#pragma unroll
    for (int i = 0; i < NRED; ++i)
        tot[i] = red[0][cg][i] + red[1][cg][i] + red[2][cg][i] + red[3][cg][i];

    if constexpr (QN) {  // the sums of the normalised k and q
        const float ik = inv_norm(tot[9]), iq = inv_norm(tot[10]);
#pragma unroll
        for (int j = 0; j < 4; ++j) { tot[j] *= ik; tot[4 + j] *= iq; }
        tot[8] *= ik * iq;
#pragma unroll
        for (int r = 0; r < RPG; ++r) kk[r] *= ik;
    }
    // correct: e = beta (v - vh); read: o = scale (p + e (k.q))
    float e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = b * (vv[j] - tot[j]);
    if (rg == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[(size_t)unit * DV + cg * 4 + j] = from_f32<Tin>(scale * (tot[4 + j] + e[j] * tot[8]));
    }
    // write: S = S~ + k e^T, back in place, non-temporal
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        float4 w;
        w.x = s[r].x + kk[r] * e[0];
        w.y = s[r].y + kk[r] * e[1];
        w.z = s[r].z + kk[r] * e[2];
        w.w = s[r].w + kk[r] * e[3];
        const f32x4 t = {w.x, w.y, w.z, w.w};
        __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(S + (size_t)(row0 + r) * DV + cg * 4));
    }
}

template <typename Tin, int DK, int DV>
static hipError_t launch_step_t(const StepArgs& a, hipStream_t stream) {
    const int units = a.N * a.H;
    if (a.fuse & FUSE_QK_L2NORM)
        hipLaunchKernelGGL((recurrent_step_kernel<Tin, DK, DV, true>), dim3(units), dim3(256), 0,
                           stream, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                           static_cast<const Tin*>(a.v), a.alpha, a.beta, a.state,
                           static_cast<Tin*>(a.o), a.scale, a.gate, a.fuse);
    else
        hipLaunchKernelGGL((recurrent_step_kernel<Tin, DK, DV, false>), dim3(units), dim3(256), 0,
                           stream, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                           static_cast<const Tin*>(a.v), a.alpha, a.beta, a.state,
                           static_cast<Tin*>(a.o), a.scale, a.gate, a.fuse);
    return hipGetLastError();
}

template <typename Tin>
static hipError_t launch_step_dt(const StepArgs& a, hipStream_t stream) {
    if (a.dk == 128 && a.dv == 128) return launch_step_t<Tin, 128, 128>(a, stream);
    if (a.dk == 128 && a.dv == 64) return launch_step_t<Tin, 128, 64>(a, stream);
    if (a.dk == 64 && a.dv == 128) return launch_step_t<Tin, 64, 128>(a, stream);
    return launch_step_t<Tin, 64, 64>(a, stream);
}

hipError_t launch_recurrent_step(const StepArgs& a, hipStream_t stream) {
    if (a.N * a.H == 0) return hipSuccess;
    return a.bf16 ? launch_step_dt<bf16_t>(a, stream) : launch_step_dt<float>(a, stream);
}

}  // namespace kda
