// backward.hip -- gradients of the KDA recurrence (the chunk-wise forward's
// outputs o and final state with respect to q, k, v, alpha, beta and the
// initial state).
//
// Method: the chain rule through the four steps of each token in reverse
// order (forget S~ = Diag(alpha_t) S, predict vh = S~^T k_t, correct and
// write S_t = S~ + beta_t k_t (v_t - vh)^T, read o_t = scale S_t^T q_t;
// "Kimi Delta Attention", section "KDA 的更新式", with the order of
// bugfactory.tech news 3610, second to fourth paragraphs).  With dS the
// gradient of S_t and e = beta_t (v_t - vh), one token back is
//   dq_t = scale S_t do_t,            dS += scale q_t do_t^T,
//   dk_t = dS e + S~ dvh,             de = dS^T k_t,
//   dbeta_t = de . (v_t - vh),        dv_t = beta_t de,   dvh = -beta_t de,
//   dS~ = dS + k_t dvh^T,             dalpha_t = rowsum(dS~ (.) S_{t-1}),
//   dS_{t-1} = Diag(alpha_t) dS~.
// The reverse sweep needs S_{t-1} of every token.  A first forward sweep
// stores the state at the start of every 16-token block (workspace); the
// reverse sweep then, block by block from the last, recomputes the block's
// 16 states forward from its checkpoint into a workspace buffer, with the
// residuals v - vh in LDS, and walks the block backwards.
//
// Layout: one workgroup per (sequence, head) unit, dk/16 waves.  Lane l of
// wave w owns state row w*16 + l%16 and the dv/4 columns of group l/16, so a
// sum over columns (dq, dk, dalpha, dbeta) stays within the lane and two
// cross-lane steps, and a sum over rows (vh, de) takes four DPP steps inside
// the 16-lane row and one pass through LDS across the waves.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int BBLK = 16;  // tokens per checkpoint block

struct BwdParams {
    const void *q, *k, *v, *dout;
    const float *alpha, *beta, *s0, *dsT;
    float *dq, *dk, *dv, *dalpha, *dbeta, *ds0;
    const int* cu_seqlens;
    float* ckpt;   // [slots per head][H][dk][dv]
    float* sbuf;   // [units][BBLK][dk][dv]
    int B, T, H, units;
    float scale;
};

// sum over the 16 lanes of a DPP row: every lane ends with the total
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));   // xor 1
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));   // xor 2
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false));  // half mirror
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, false));  // mirror
    return x;
}
// sum over the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float groups4_sum(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

template <typename Tin, int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 16)) void backward_kernel(BwdParams p) {
    constexpr int NW = DK / 16;   // waves, 16 state rows each
    constexpr int CPL = DV / 4;   // columns per lane
    __shared__ __align__(16) float part[NW][DV];     // per-wave partial sums over rows
    __shared__ __align__(16) float red[DV];          // their total
    __shared__ __align__(16) float resid[BBLK][DV];  // v - vh of the block tokens

    const int unit = blockIdx.x;
    const int H = p.H, seq = unit / H, h = unit % H;
    long t0;
    int len;
    if (p.cu_seqlens) {
        t0 = p.cu_seqlens[seq];
        len = p.cu_seqlens[seq + 1] - (int)t0;
    } else {
        t0 = (long)seq * p.T;
        len = p.T;
    }
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int row = w * 16 + (l & 15), cg = l >> 4, c0 = cg * CPL;
    const Tin* __restrict__ gq = static_cast<const Tin*>(p.q);
    const Tin* __restrict__ gk = static_cast<const Tin*>(p.k);
    const Tin* __restrict__ gv = static_cast<const Tin*>(p.v);
    const Tin* __restrict__ gdo = static_cast<const Tin*>(p.dout);
    const size_t sunit = (size_t)unit * DK * DV + (size_t)row * DV + c0;  // this lane's state run
    // checkpoint slots of this sequence: cu/BBLK + seq keeps the sequences'
    // runs of ceil(len/BBLK) slots apart
    const long slot0 = t0 / BBLK + seq;
    auto ckpt_at = [&](int blk) {
        return p.ckpt + ((size_t)(slot0 + blk) * H + h) * DK * DV + (size_t)row * DV + c0;
    };
    float* sb = p.sbuf + (size_t)unit * BBLK * DK * DV + (size_t)row * DV + c0;

    auto ld_cols = [&](const Tin* base, float (&x)[CPL]) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) x[j] = to_f32(base[c0 + j]);
    };
    auto ld_run = [&](const float* src, float (&x)[CPL]) {
#pragma unroll
        for (int j = 0; j < CPL; j += 4) {
            const float4 f = *reinterpret_cast<const float4*>(src + j);
            x[j] = f.x; x[j + 1] = f.y; x[j + 2] = f.z; x[j + 3] = f.w;
        }
    };
    auto st_run = [&](float* dst, const float (&x)[CPL]) {
#pragma unroll
        for (int j = 0; j < CPL; j += 4)
            *reinterpret_cast<float4*>(dst + j) = make_float4(x[j], x[j + 1], x[j + 2], x[j + 3]);
    };
    // x[j] <- sum over the dk rows of x[j] (column c0 + j); two barriers
    auto col_sum = [&](float (&x)[CPL]) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) x[j] = row16_sum(x[j]);
        if ((l & 15) == 0) st_run(&part[w][c0], x);
        __syncthreads();
        for (int c = tid; c < DV; c += 64 * NW) {
            float s = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) s += part[ww][c];
            red[c] = s;
        }
        __syncthreads();
        ld_run(&red[c0], x);
    };
    // one forward token step on this lane's run; r receives v - vh
    auto fwd_step = [&](float (&S)[CPL], long tok, float (&r)[CPL]) {
        const size_t th = (size_t)tok * H + h;
        const float kr = to_f32(gk[th * DK + row]);
        const float ar = p.alpha[th * DK + row];
        const float b = p.beta[th];
        float vv[CPL], x[CPL];
        ld_cols(gv + th * DV, vv);
#pragma unroll
        for (int j = 0; j < CPL; ++j) { S[j] *= ar; x[j] = S[j] * kr; }
        col_sum(x);  // vh
#pragma unroll
        for (int j = 0; j < CPL; ++j) { r[j] = vv[j] - x[j]; S[j] += kr * (b * r[j]); }
    };

    const int nblk = (len + BBLK - 1) / BBLK;
    float S[CPL];
    if (p.s0) ld_run(p.s0 + sunit, S);
    else {
#pragma unroll
        for (int j = 0; j < CPL; ++j) S[j] = 0.f;
    }
    // sweep 1: checkpoints at the block starts
    for (int t = 0; t < len; ++t) {
        if (t % BBLK == 0) st_run(ckpt_at(t / BBLK), S);
        float r[CPL];
        fwd_step(S, t0 + t, r);
    }
    // sweep 2: blocks from the last, each recomputed and then reversed
    float dS[CPL];
    if (p.dsT) ld_run(p.dsT + sunit, dS);
    else {
#pragma unroll
        for (int j = 0; j < CPL; ++j) dS[j] = 0.f;
    }
    const float sc = p.scale;
    for (int blk = nblk - 1; blk >= 0; --blk) {
        const int tb = blk * BBLK, nt = min(BBLK, len - tb);
        ld_run(ckpt_at(blk), S);
        for (int tt = 0; tt < nt; ++tt) {
            st_run(sb + (size_t)tt * DK * DV, S);  // S_{t-1} of token tb + tt
            float r[CPL];
            fwd_step(S, t0 + tb + tt, r);
            if (w == 0 && (l & 15) == 0) st_run(&resid[tt][c0], r);
        }
        __syncthreads();
        for (int tt = nt - 1; tt >= 0; --tt) {
            const long tok = t0 + tb + tt;
            const size_t th = (size_t)tok * H + h;
            const float kr = to_f32(gk[th * DK + row]);
            const float qr = to_f32(gq[th * DK + row]);
            const float ar = p.alpha[th * DK + row];
            const float b = p.beta[th];
            float sp[CPL], r[CPL], dov[CPL];
            ld_run(sb + (size_t)tt * DK * DV, sp);
            ld_run(&resid[tt][c0], r);
            ld_cols(gdo + th * DV, dov);
            float st[CPL], e[CPL];
            float dq = 0.f, dkr = 0.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                st[j] = ar * sp[j];
                e[j] = b * r[j];
                dq += (st[j] + kr * e[j]) * dov[j];     // S_t do_t
                dS[j] += sc * qr * dov[j];
                dkr += dS[j] * e[j];
            }
            float de[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) de[j] = dS[j] * kr;
            col_sum(de);  // de = dS^T k_t
            float db = 0.f, da = 0.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                db += de[j] * r[j];
                const float dvh = -b * de[j];
                const float dst = dS[j] + kr * dvh;
                dkr += st[j] * dvh;
                da += dst * sp[j];
                dS[j] = ar * dst;
            }
            dq = groups4_sum(dq);
            dkr = groups4_sum(dkr);
            da = groups4_sum(da);
            db = groups4_sum(db);
            if (cg == 0) {
                p.dq[th * DK + row] = sc * dq;
                p.dk[th * DK + row] = dkr;
                p.dalpha[th * DK + row] = da;
            }
            if (w == 0 && (l & 15) == 0) {
#pragma unroll
                for (int j = 0; j < CPL; ++j) p.dv[th * DV + c0 + j] = b * de[j];
            }
            if (tid == 0) p.dbeta[th] = db;
        }
        __syncthreads();  // resid is rewritten by the next block
    }
    st_run(p.ds0 + sunit, dS);
}

template <typename Tin, int DK, int DV>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
    hipLaunchKernelGGL((backward_kernel<Tin, DK, DV>), dim3(p.units), dim3(64 * (DK / 16)), 0,
                       stream, p);
    return hipGetLastError();
}

template <typename Tin>
hipError_t launch_bwd_dt(const BwdParams& p, int dk, int dv, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_bwd_t<Tin, 128, 128>(p, stream);
    if (dk == 128 && dv == 64) return launch_bwd_t<Tin, 128, 64>(p, stream);
    if (dk == 64 && dv == 128) return launch_bwd_t<Tin, 64, 128>(p, stream);
    return launch_bwd_t<Tin, 64, 64>(p, stream);
}

}  // namespace

size_t backward_workspace_bytes(long tokens_total, int nseq, int H, int dk, int dv) {
    const size_t slots = (size_t)((tokens_total + BBLK - 1) / BBLK + nseq + 1);
    const size_t ck = slots * H * dk * dv * 4;
    const size_t sb = (size_t)nseq * H * BBLK * dk * dv * 4;
    return (ck + 255) / 256 * 256 + (sb + 255) / 256 * 256;
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
    const int nseq = a.cu_seqlens ? a.num_seqs : a.B;
    const int units = nseq * a.H;
    if (units == 0) return hipSuccess;
    const long tokens = a.cu_seqlens ? a.T : (long)a.B * a.T;
    const size_t slots = (size_t)((tokens + BBLK - 1) / BBLK + nseq + 1);
    const size_t ck = (slots * a.H * a.dk * a.dv * 4 + 255) / 256 * 256;
    BwdParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.dout = a.dout;
    p.alpha = a.alpha; p.beta = a.beta; p.s0 = a.s0; p.dsT = a.dsT;
    p.dq = a.g_q; p.dk = a.g_k; p.dv = a.g_v; p.dalpha = a.g_alpha; p.dbeta = a.g_beta;
    p.ds0 = a.g_s0;
    p.cu_seqlens = a.cu_seqlens;
    p.ckpt = static_cast<float*>(a.workspace);
    p.sbuf = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + ck);
    p.B = a.B; p.T = a.T; p.H = a.H; p.units = units;
    p.scale = a.scale;
    return a.bf16 ? launch_bwd_dt<bf16_t>(p, a.dk, a.dv, stream)
                   : launch_bwd_dt<float>(p, a.dk, a.dv, stream);
}

}  // namespace kda
