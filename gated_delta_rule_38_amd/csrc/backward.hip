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
// stores the state at the start of every 8-token block (workspace); the
// reverse sweep then, block by block from the last, recomputes the block's
// 8 states forward from its checkpoint into registers, with the residuals
// v - vh in LDS, and walks the block backwards.  Both sweeps issue each token's
// input loads a few steps ahead.
//
// Layout: one workgroup per (sequence, head) unit and slice of DVS value
// columns (the columns of S evolve independently), dk/16 waves.  Lane l of
// wave w owns state row w*16 + l%16 and the DVS/4 columns of group l/16, so
// a sum over the slice's columns (dq, dk, dalpha, dbeta) stays within the
// lane and two cross-lane steps, and a sum over rows (vh, de) takes four DPP
// steps inside the 16-lane row and one pass through LDS across the waves.
// The slices of a unit add their column sums into the zeroed dq, dk, dalpha
// and dbeta with float atomics; dv and the initial-state gradient are the
// slice's own columns.
#include <algorithm>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int BBLK = 8;  // tokens per checkpoint block
// tokens whose input loads are in flight ahead of their step in the first
// sweep (fp32 inputs take more registers: one ahead keeps two workgroups per
// compute unit)
template <typename Tin>
constexpr int prefetch_depth() { return sizeof(Tin) == 2 ? 6 : 1; }
constexpr int PD2 = 2;  // the same in the second sweep (whole blocks)

struct BwdParams {
    const void *q, *k, *v, *dout;
    const float *alpha, *beta, *s0, *dsT;
    float *dq, *dk, *dv, *dalpha, *dbeta, *ds0;
    const int* cu_seqlens;
    float* ckpt;   // [slots per head][H][dk][dv]
    int B, T, H, units, nslice;
    float scale;
};

__global__ void zero_kernel(float* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

// sum over the 16 lanes of a DPP row: every lane ends with the total
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));   // xor 1
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));   // xor 2
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false));  // half mirror
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, false));  // mirror
    return x;
}
// Workgroup barrier that orders LDS only.  The waves exchange nothing but LDS
// data; every global location a lane reads back (checkpoints, block states)
// it wrote itself, and the gradient sums are atomics.  A full barrier would
// also wait for every global store and atomic in flight, and with them for
// the next token's loads issued ahead.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// sum over the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float groups4_sum(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

template <typename Tin, int DK, int DV, int DVS>
__global__ __launch_bounds__(64 * (DK / 16), 4) void backward_kernel(BwdParams p) {
    constexpr int NW = DK / 16;   // waves, 16 state rows each
    constexpr int CPL = DVS / 4;  // columns per lane
    __shared__ __align__(16) float part[2][NW][DVS];  // per-wave partial sums over rows
    __shared__ __align__(16) float resid[BBLK][DVS];  // v - vh of the block tokens

    const int unit = blockIdx.x / p.nslice, slice = blockIdx.x % p.nslice;
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
    const int row = w * 16 + (l & 15), cg = l >> 4, cs = cg * CPL;  // column in the slice
    const int c0 = slice * DVS + cs;                                  // column in the state
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
    // x[j] <- sum over the dk rows of x[j] (column c0 + j): one barrier, the
    // partials double-buffered so the next sum cannot overwrite them early
    int rpar = 0;
    auto col_sum = [&](float (&x)[CPL]) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) x[j] = row16_sum(x[j]);
        if ((l & 15) == 0) st_run(&part[rpar][w][cs], x);
        lds_barrier();
        float y[CPL];
        ld_run(&part[rpar][0][cs], x);
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) {
            ld_run(&part[rpar][ww][cs], y);
#pragma unroll
            for (int j = 0; j < CPL; ++j) x[j] += y[j];
        }
        rpar ^= 1;
    };
    // A token's inputs for this lane, kept as loaded (bf16 unconverted) and
    // issued PD steps ahead of their use, so that a token step does not wait
    // for a load's latency (the block loops are unrolled: every index into
    // the per-token arrays is a constant and nothing is copied).
    // (CPL = 4 columns: one 8-byte load in bf16, 16 bytes in fp32)
    typedef Tin Tin4 __attribute__((ext_vector_type(4)));
    static_assert(CPL == 4, "four columns per lane");
    struct FIn { Tin kr; float ar, b; Tin4 vv; };
    struct QIn { Tin kr, qr; float ar, b; Tin4 dov; };  // the reverse step's
    auto ld_fin = [&](long tok, FIn& f) {
        const size_t th = (size_t)tok * H + h;
        f.kr = gk[th * DK + row];
        f.ar = p.alpha[th * DK + row];
        f.b = p.beta[th];
        f.vv = *reinterpret_cast<const Tin4*>(gv + th * DV + c0);
    };
    auto ld_qin = [&](long tok, QIn& g) {
        const size_t th = (size_t)tok * H + h;
        g.kr = gk[th * DK + row];
        g.qr = gq[th * DK + row];
        g.ar = p.alpha[th * DK + row];
        g.b = p.beta[th];
        g.dov = *reinterpret_cast<const Tin4*>(gdo + th * DV + c0);
    };
    // one forward token step on this lane's run; r receives v - vh
    auto fwd_step = [&](float (&S)[CPL], const FIn& f, float (&r)[CPL]) {
        const float kr = to_f32(f.kr);
        float x[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) { S[j] *= f.ar; x[j] = S[j] * kr; }
        col_sum(x);  // vh
#pragma unroll
        for (int j = 0; j < CPL; ++j) { r[j] = to_f32(f.vv[j]) - x[j]; S[j] += kr * (f.b * r[j]); }
    };

    const int nblk = (len + BBLK - 1) / BBLK;
    float S[CPL];
    if (p.s0) ld_run(p.s0 + sunit, S);
    else {
#pragma unroll
        for (int j = 0; j < CPL; ++j) S[j] = 0.f;
    }
    // sweep 1: checkpoints at the block starts (the loops over a block are
    // unrolled so that every index is a constant; nt is uniform)
    for (int blk = 0; blk < nblk; ++blk) {
        const int tb = blk * BBLK, nt = min(BBLK, len - tb);
        constexpr int PD = prefetch_depth<Tin>();
        FIn f[BBLK];
#pragma unroll
        for (int tt = 0; tt < PD; ++tt)
            if (tt < nt) ld_fin(t0 + tb + tt, f[tt]);
        st_run(ckpt_at(blk), S);
#pragma unroll
        for (int tt = 0; tt < BBLK; ++tt) {
            if (tt < nt) {
                if (tt + PD < BBLK && tt + PD < nt) ld_fin(t0 + tb + tt + PD, f[tt + PD]);
                float r[CPL];
                fwd_step(S, f[tt], r);
            }
        }
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
        // the block's states S_{t-1}, in registers (every index into SB is a
        // constant once the block loops are unrolled)
        float SB[BBLK][CPL];
        auto rec_step = [&](int tt, const FIn& fi) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) SB[tt][j] = S[j];
            float r[CPL];
            fwd_step(S, fi, r);
            if (w == 0 && (l & 15) == 0) st_run(&resid[tt][cs], r);
        };
        auto rev_step = [&](int tt, const QIn& bc) {
            const long tok = t0 + tb + tt;
            const size_t th = (size_t)tok * H + h;
            const float kr = to_f32(bc.kr), qr = to_f32(bc.qr), ar = bc.ar, b = bc.b;
            const float(&sp)[CPL] = SB[tt];
            float dov[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) dov[j] = to_f32(bc.dov[j]);
            float r[CPL];
            ld_run(&resid[tt][cs], r);
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
                atomicAdd(p.dq + th * DK + row, sc * dq);
                atomicAdd(p.dk + th * DK + row, dkr);
                atomicAdd(p.dalpha + th * DK + row, da);
            }
            if (w == 0 && (l & 15) == 0) {
#pragma unroll
                for (int j = 0; j < CPL; ++j) p.dv[th * DV + c0 + j] = b * de[j];
            }
            if (tid == 0) atomicAdd(p.dbeta + th, db);
        };
        if (nt == BBLK) {
            // a whole block: every token's loads issued PD2 steps ahead into
            // slots with constant indices, each defined once
            FIn f[BBLK];
            QIn g[BBLK];
#pragma unroll
            for (int tt = 0; tt < PD2; ++tt) ld_fin(t0 + tb + tt, f[tt]);
#pragma unroll
            for (int tt = 0; tt < BBLK; ++tt) {
                if (tt + PD2 < BBLK) ld_fin(t0 + tb + tt + PD2, f[tt + PD2]);
                if (tt >= BBLK - PD2) {  // the reverse walk's first inputs
                    const int tr = 2 * BBLK - PD2 - 1 - tt;
                    ld_qin(t0 + tb + tr, g[tr]);
                }
                rec_step(tt, f[tt]);
            }
            lds_barrier();
#pragma unroll
            for (int tt = BBLK - 1; tt >= 0; --tt) {
                if (tt >= PD2) ld_qin(t0 + tb + tt - PD2, g[tt >= PD2 ? tt - PD2 : 0]);
                rev_step(tt, g[tt]);
            }
        } else {
            // the short last block of a sequence: loads one step ahead
            FIn fc, fn;
            ld_fin(t0 + tb, fn);
#pragma unroll
            for (int tt = 0; tt < BBLK; ++tt) {
                if (tt < nt) {
                    fc = fn;
                    if (tt + 1 < nt) ld_fin(t0 + tb + tt + 1, fn);
                    rec_step(tt, fc);
                }
            }
            lds_barrier();
            QIn bc, bn;
            ld_qin(t0 + tb + nt - 1, bn);
#pragma unroll
            for (int tt = BBLK - 1; tt >= 0; --tt) {
                if (tt < nt) {
                    bc = bn;
                    if (tt > 0) ld_qin(t0 + tb + tt - 1, bn);
                    rev_step(tt, bc);
                }
            }
        }
        lds_barrier();  // resid is rewritten by the next block
    }
    st_run(p.ds0 + sunit, dS);
}

template <typename Tin, int DK, int DV>
hipError_t launch_bwd_t(BwdParams p, long tokens, hipStream_t stream) {
    constexpr int DVS = 16;  // value columns per workgroup (4 per lane)
    p.nslice = DV / DVS;
    // the column sums are accumulated: clear dq, dk, dalpha (tokens*H*dk each) and dbeta
    const size_t nk = (size_t)tokens * p.H * DK, nb = (size_t)tokens * p.H;
    // (no tokens: nothing to clear, and a grid of zero workgroups is not a launch)
    if (nk > 0) {
        float* zs[] = {p.dq, p.dk, p.dalpha};
        for (float* z : zs) {
            hipLaunchKernelGGL(zero_kernel,
                               dim3((unsigned)std::min<size_t>((nk + 255) / 256, 4096)), dim3(256),
                               0, stream, z, nk);
        }
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)std::min<size_t>((nb + 255) / 256, 4096)),
                           dim3(256), 0, stream, p.dbeta, nb);
    }
    hipLaunchKernelGGL((backward_kernel<Tin, DK, DV, DVS>), dim3(p.units * p.nslice),
                       dim3(64 * (DK / 16)), 0, stream, p);
    return hipGetLastError();
}

template <typename Tin>
hipError_t launch_bwd_dt(const BwdParams& p, int dk, int dv, long tokens, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_bwd_t<Tin, 128, 128>(p, tokens, stream);
    if (dk == 128 && dv == 64) return launch_bwd_t<Tin, 128, 64>(p, tokens, stream);
    if (dk == 64 && dv == 128) return launch_bwd_t<Tin, 64, 128>(p, tokens, stream);
    return launch_bwd_t<Tin, 64, 64>(p, tokens, stream);
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
    const int nseq = a.cu_seqlens ? a.num_seqs : a.B;
    const int units = nseq * a.H;
    if (units == 0) return hipSuccess;
    const long tokens = a.cu_seqlens ? a.T : (long)a.B * a.T;
    BwdParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.dout = a.dout;
    p.alpha = a.alpha; p.beta = a.beta; p.s0 = a.s0; p.dsT = a.dsT;
    p.dq = a.g_q; p.dk = a.g_k; p.dv = a.g_v; p.dalpha = a.g_alpha; p.dbeta = a.g_beta;
    p.ds0 = a.g_s0;
    p.cu_seqlens = a.cu_seqlens;
    p.ckpt = static_cast<float*>(a.workspace);
    p.B = a.B; p.T = a.T; p.H = a.H; p.units = units;
    p.scale = a.scale;
    return a.bf16 ? launch_bwd_dt<bf16_t>(p, a.dk, a.dv, tokens, stream)
                   : launch_bwd_dt<float>(p, a.dk, a.dv, tokens, stream);
}

}  // namespace kda
