// gdn2_step.hip -- one-token Gated DeltaNet-2 decode step, state updated in
// place.
//
// Method: "线性注意力机制：从标准注意力到 Gated DeltaNet-2" (jindou-blog),
// section 4 "Gated DeltaNet-2：解耦擦除与写入": the delta rule's one write
// strength is split into an erase gate e_t and a write gate w_t, each a vector
// over the key channels.  Read with the forget gate of KDA kept, one token is
//   S~  = Diag(alpha_t) S             forget
//   vh  = S~^T k_t                    predict
//   S_t = S~ - (e_t . k_t) vh^T + (w_t . k_t) v_t^T    erase, write
//   o_t = scale S_t^T q_t             read
// (e_t = w_t = beta_t reproduces the KDA step; the token-by-token mode is the
// "fused recurrent" mode of bugfactory.tech news 3610, fifth paragraph).
//
// The step is HBM-bound like the KDA step (one pass over the fp32 state, in and
// out) and uses the same layout: one 256-thread workgroup per (sequence, head),
// thread (rg, cg) holding rows rg*RPG.. of value columns 4cg..4cg+3 as float4
// registers.  The reductions over the key dimension (vh, p = S~^T q, and the
// two gated dot products (e.k).q and (w.k).q) share one pass, and the read
// needs no second pass: o = scale (p - ((e.k).q) vh + ((w.k).q) v), which equals
// scale S_t^T q.  The new state leaves with non-temporal stores.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <typename Tin, int DK, int DV>
__global__ __launch_bounds__(256) void gdn2_step_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ erase,
    const float* __restrict__ write, float* __restrict__ state, Tin* __restrict__ o,
    float scale) {
    constexpr int NCG = DV / 4;      // float4 column groups
    constexpr int NRG = 256 / NCG;   // row groups
    constexpr int RPG = DK / NRG;    // rows per thread
    constexpr int NRED = 10;         // 4 x vh, 4 x p, (e.k).q, (w.k).q
    static_assert(NCG <= 64 && 64 % NCG == 0 && RPG >= 1, "shape");

    __shared__ float red[4][NCG][NRED + 1];

    const int unit = blockIdx.x;  // sequence * H + head
    const int tid = threadIdx.x;
    const int cg = tid % NCG;
    const int rg = tid / NCG;
    const int row0 = rg * RPG;
    float* __restrict__ S = state + (size_t)unit * DK * DV;

    float4 s[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r)
        s[r] = *reinterpret_cast<const float4*>(S + (size_t)(row0 + r) * DV + cg * 4);

    float a[RPG], kk[RPG], qq[RPG], ek[RPG], wk[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        const size_t i = (size_t)unit * DK + row0 + r;
        a[r] = alpha ? alpha[i] : 1.f;
        kk[r] = to_f32(k[i]);
        qq[r] = to_f32(q[i]);
        ek[r] = erase[i] * kk[r];
        wk[r] = write[i] * kk[r];
    }
    float vv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vv[j] = to_f32(v[(size_t)unit * DV + cg * 4 + j]);

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
        part[8] += ek[r] * qq[r];
        part[9] += wk[r] * qq[r];
    }
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

    if (rg == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[(size_t)unit * DV + cg * 4 + j] =
                from_f32<Tin>(scale * (tot[4 + j] - tot[8] * tot[j] + tot[9] * vv[j]));
    }
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        const f32x4 t = {s[r].x - ek[r] * tot[0] + wk[r] * vv[0],
                         s[r].y - ek[r] * tot[1] + wk[r] * vv[1],
                         s[r].z - ek[r] * tot[2] + wk[r] * vv[2],
                         s[r].w - ek[r] * tot[3] + wk[r] * vv[3]};
        __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(S + (size_t)(row0 + r) * DV + cg * 4));
    }
}

template <typename Tin, int DK, int DV>
static hipError_t launch_gdn2_step_t(const Gdn2StepArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((gdn2_step_kernel<Tin, DK, DV>), dim3(a.N * a.H), dim3(256), 0, stream,
                       static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                       static_cast<const Tin*>(a.v), a.alpha, a.erase, a.write, a.state,
                       static_cast<Tin*>(a.o), a.scale);
    return hipGetLastError();
}

template <typename Tin>
static hipError_t launch_gdn2_step_dt(const Gdn2StepArgs& a, hipStream_t stream) {
    if (a.dk == 128 && a.dv == 128) return launch_gdn2_step_t<Tin, 128, 128>(a, stream);
    if (a.dk == 128 && a.dv == 64) return launch_gdn2_step_t<Tin, 128, 64>(a, stream);
    if (a.dk == 64 && a.dv == 128) return launch_gdn2_step_t<Tin, 64, 128>(a, stream);
    return launch_gdn2_step_t<Tin, 64, 64>(a, stream);
}

hipError_t launch_gdn2_step(const Gdn2StepArgs& a, hipStream_t stream) {
    if (a.N * a.H == 0) return hipSuccess;
    return a.bf16 ? launch_gdn2_step_dt<bf16_t>(a, stream) : launch_gdn2_step_dt<float>(a, stream);
}

}  // namespace kda
