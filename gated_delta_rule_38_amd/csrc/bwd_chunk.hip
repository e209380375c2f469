// bwd_chunk.hip -- gradients of the chunk-wise KDA forward in the chunk form,
// on gfx950 matrix cores (bf16 operands, fp32 accumulation).
//
// Method: the chain rule through the chunk form of the update ("Kimi Delta
// Attention", section "KDA 的更新式"; the chunk-wise mode of bugfactory.tech
// news 3610, fifth paragraph, which serves training, with matrix products
// inside a chunk and the state carried between chunks as on the kongchang.com
// page, section "硬件效率的优化策略").  The identities are derived from the
// update (the pages print none).  A first launch, the chunk-wise forward with
// checkpoints, stores the state at the start of every 64-token chunk.  This
// kernel then walks each unit's chunks from the last to the first with the
// gradient dS of the chunk-end state in registers.  With the forward's
// operands of a chunk (P_r the running product of alpha from the chunk start,
// Pm = P_31, Pn = P_63, Kr = K P/Pm, Qr = Q P/Pm, Kc = K Pm/P, SP = Pm S0,
// A = tril_-1(Kr Kc^T), M = tril(Qr Kc^T), T' = (I + Diag(beta) A)^{-1},
// X = V - Kr SP, Y = beta X, U = T' Y), one chunk back is
//   dW  = (Pn/Pm) dS,                 dU  = scale M^T dO + Kc dW
//   dY  = T'^T dU,                     dX  = beta dY,  dv = dX
//   G   = dY U^T,  dA = -Diag(beta) G (strictly lower),  dM = scale dO U^T (lower)
//   dbeta = rowsum(dY X) - rowsum(G A) (strictly lower part)
//   dQr = scale dO SP^T + dM Kc,       dKr = -dX SP^T + dA Kc
//   dKc = U dW^T + dA^T Kr + dM^T Qr
//   dq  = dQr P/Pm,  dk = dKr P/Pm + dKc Pm/P
//   dlogP_r = dKr Kr - dKc Kc + dQr Qr (+ rowsum(dS S_C) at the last row)
//   dalpha_t = sum_{r >= t} dlogP_r / alpha_t
//   dS <- Pn dS + Pm (scale Qr^T dO - Kr^T dX)
// (the mid-chunk reference Pm cancels out of every product, so its own
// derivative terms sum to zero and are left out).
//
// Work decomposition as in the forward: one workgroup of four waves owns one
// (unit, 32-column value slice); the columns of dS evolve independently, so
// the chain needs no exchange between slices.  dv and dS_0 are each slice's
// own columns.  dq, dk, dalpha and dbeta sum over the value columns: slice 0
// writes its part into the outputs and every other slice into a plane of its
// own in the workspace, each element once; a last pass adds the planes in
// slice order, so the gradients are the same bit for bit from run to run.  A chunk runs in
// eight phases separated by workgroup barriers; the LDS regions of the phases
// overlay one another.
#include <algorithm>

#include "chunk_walk.h"

namespace kda {

namespace {

constexpr int BW_NTH = 256;
// half-chunk decay product below which a chunk's gradients are taken token by token
constexpr float BW_DECAY_FLOOR = 0x1p-12f;

struct BwParams {
    KParams base;          // q, k, v, alpha, beta, cu_seqlens, order, B, T, H, dv, mapping, scale
    const void* dout;      // [tokens, H, dv] bf16
    const float* ckpt;     // chunk-start states (the forward with checkpoints)
    const float* dsT;      // [units, dk, dv] or NULL
    float *dq, *dk, *dv, *dalpha, *dbeta, *ds0;
    // partial sums of value-column slices 1.. (slice 0 writes the outputs):
    // slice j's dq, dk, dalpha ([tokens, H, dk] each) and dbeta ([tokens, H],
    // padded to nb) start at part + (j - 1) * (3 nk + nb)
    float* part;
    size_t nk, nb;
};

// Where value-column slice jt writes its parts of dq, dk, dalpha and dbeta.
struct GradOut {
    float *dq, *dk, *da, *db;
};
__device__ __forceinline__ GradOut grad_out(const BwParams& bp, int jt) {
    if (jt == 0) return {bp.dq, bp.dk, bp.dalpha, bp.dbeta};
    float* b = bp.part + (size_t)(jt - 1) * (3 * bp.nk + bp.nb);
    return {b, b + bp.nk, b + 2 * bp.nk, b + 3 * bp.nk};
}

template <int DK, int DVT>
struct BwLayout {
    static constexpr int ES = 2;
    static constexpr int LDK = DK + 8;    // [token][channel]
    static constexpr int LDC = CH + 8;    // [*][token]
    static constexpr int LDV = DVT + 8;   // [*][value column]
    static constexpr int LDD = 24;
    static constexpr int LDL = 20;
    static constexpr int NJT = DVT / 16;
    static constexpr int NCT = DK / 16;
    static constexpr int NST = NCT * NJT;
    static constexpr int STW = (NST + 3) / 4;
    static_assert(NJT <= 2, "slice width");
    // persistent (phases 1-7)
    static constexpr size_t oSPr = 0;                                   // [DK][LDV] SP
    static constexpr size_t odWr = oSPr + (size_t)DK * LDV * ES;        // [DK][LDV] dW
    static constexpr size_t odOr = odWr + (size_t)DK * LDV * ES;        // [CH][LDV] dO
    static constexpr size_t oBeta = odOr + (size_t)CH * LDV * ES;       // fp32 [64]
    static constexpr size_t oTot = oBeta + 256;                         // fp32 [4][DK]
    static constexpr size_t odlPn = oTot + (size_t)4 * DK * 4;          // fp32 [2][DK]
    static constexpr size_t oDb1 = odlPn + (size_t)2 * DK * 4;          // fp32 [64]
    static constexpr size_t oDb2 = oDb1 + 256;                          // fp32 [10][16]
    static constexpr size_t endP = (oDb2 + 640 + 255) / 256 * 256;
    // region 2 (phases 1-6)
    static constexpr size_t odOT = endP;                                // [DVT][LDC] dO^T
    static constexpr size_t oLo = odOT + (size_t)DVT * LDC * ES;        // [CH][LDC] beta A, off-diagonal
    static constexpr size_t oLd = oLo + (size_t)CH * LDC * ES;          // fp32 [4][16][LDL]
    static constexpr size_t oMT = oLd + (size_t)4 * 16 * LDL * 4;       // [CH][LDC] M^T
    static constexpr size_t oYT = oMT + (size_t)CH * LDC * ES;          // [DVT][LDC] Y^T
    static constexpr size_t endR2 = oYT + (size_t)DVT * LDC * ES;
    //   phases 4-6 over Lo .. MT
    static constexpr size_t oUr = oLo;                                  // [CH][LDV] U
    static constexpr size_t odYr = oUr + (size_t)CH * LDV * ES;         // [CH][LDV] dY
    static constexpr size_t odXr = odYr + (size_t)CH * LDV * ES;        // [CH][LDV] dX
    static constexpr size_t odXT = odXr + (size_t)CH * LDV * ES;        // [DVT][LDC] dX^T
    static_assert(odXT + (size_t)DVT * LDC * ES <= oYT, "phase 4 overlay");
    // region 1: phases 1-2
    static constexpr size_t R1 = (endR2 + 255) / 256 * 256;
    static constexpr size_t oKr = R1;                                   // [CH][LDK]
    static constexpr size_t oQr = oKr + (size_t)CH * LDK * ES;
    static constexpr size_t oKc = oQr + (size_t)CH * LDK * ES;
    static constexpr size_t oSPT = oKc + (size_t)CH * LDK * ES;         // [DVT][LDK] SP^T
    static constexpr size_t odWT = oSPT + (size_t)DVT * LDK * ES;       // [DVT][LDK] dW^T
    static constexpr size_t end1 = odWT + (size_t)DVT * LDK * ES;
    //   phases 3-4
    static constexpr size_t oTm = R1;                                   // [CH][LDC] T'
    static constexpr size_t oTmT = oTm + (size_t)CH * LDC * ES;         // [CH][LDC] T'^T
    static constexpr size_t oDr = oTmT + (size_t)CH * LDC * ES;
    static constexpr size_t oDc = oDr + (size_t)4 * 4 * 16 * LDD * ES;
    static constexpr size_t odUT = oDc + (size_t)4 * 4 * 16 * LDD * ES; // [DVT][LDC] dU^T
    static constexpr size_t end3 = odUT + (size_t)DVT * LDC * ES;
    //   phases 5-6
    static constexpr size_t oKrT = R1;                                  // [DK][LDC]
    static constexpr size_t oQrT = oKrT + (size_t)DK * LDC * ES;
    static constexpr size_t oKcT = oQrT + (size_t)DK * LDC * ES;
    static constexpr size_t odA = oKcT + (size_t)DK * LDC * ES;         // [CH][LDC] dA
    static constexpr size_t odAT = odA + (size_t)CH * LDC * ES;
    static constexpr size_t odM = odAT + (size_t)CH * LDC * ES;
    static constexpr size_t odMT = odM + (size_t)CH * LDC * ES;
    static constexpr size_t end5 = odMT + (size_t)CH * LDC * ES;
    static constexpr size_t bytes0 = end1 > end3 ? end1 : end3;
    static constexpr size_t bytes = bytes0 > end5 ? bytes0 : end5;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

template <int CPT> struct BwRow;
template <> struct BwRow<1> {
    typedef uint16_t B;
    typedef float F;
    static __device__ __forceinline__ B ldb(const bf16_t* p) { return *reinterpret_cast<const uint16_t*>(p); }
    static __device__ __forceinline__ F ldf(const float* p) { return *p; }
    static __device__ __forceinline__ void ub(B w, float* x) { x[0] = __uint_as_float(uint32_t(w) << 16); }
    static __device__ __forceinline__ void uf(F w, float* x) { x[0] = w; }
};
template <> struct BwRow<2> {
    typedef uint32_t B;
    typedef float2 F;
    static __device__ __forceinline__ B ldb(const bf16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
    static __device__ __forceinline__ F ldf(const float* p) { return *reinterpret_cast<const float2*>(p); }
    static __device__ __forceinline__ void ub(B w, float* x) {
        x[0] = __uint_as_float(w << 16);
        x[1] = __uint_as_float(w & 0xffff0000u);
    }
    static __device__ __forceinline__ void uf(F w, float* x) { x[0] = w.x; x[1] = w.y; }
};

// sum over the 16 lanes of a DPP row; every lane ends with the total
__device__ __forceinline__ float row16_total(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    return x;
}

// Exact gradients of one chunk, token by token.  The reverse sweep switches to
// this at the first chunk (from the end) that fails its range check (a
// half-chunk product of alpha below 2^-12 in some key channel) and keeps it
// down to the first chunk.  The checkpoints it starts from are exact or as
// close as the chunk-wise forward (which redoes a unit token by token below
// 2^-100).  The chain rule through one token's update
//   S~ = Diag(alpha) S_,  vh = S~^T k,  u = beta (v - vh),  S = S~ + k u^T,  o = scale S^T q
// with G = dS + scale q do^T (dS the gradient of S) gives
//   dq = scale S do,  du = G^T k,  dv = beta du,  dbeta = du . (v - vh),
//   dk = G u - beta S~ du,  dS~ = G - beta k du^T,
//   dalpha = rowsum(dS~ * S_),  dS_ = Diag(alpha) dS~,
// taken from the chunk's last token to its first.  The state before each token
// is recomputed from the chunk-start checkpoint through eight snapshots (one
// per 8 tokens) kept in LDS.  Thread (rg, c) holds rows rg*RPT.. of column c
// of the slice; dS enters and leaves in the C-layout tiles of the chunk form.
template <int DK, int DVT, int STW>
__device__ __forceinline__ void bw_token_chunk(const BwParams& bp, int seq, int h, long t0, int len,
                                               int ch, int col0, const float* ckpt, f32x4 (&dS)[STW],
                                               float* lds) {
    static_assert(DVT == 32 && BW_NTH == 256, "one 32-column slice over 256 threads");
    constexpr int NJT = DVT / 16, NST = (DK / 16) * NJT;
    constexpr int NRG = BW_NTH / DVT;  // 8 row groups
    constexpr int RPT = DK / NRG;      // rows per thread (16 or 8)
    constexpr int SNAP = 8;            // tokens per snapshot
    const KParams& p = bp.base;
    const int H = p.H, DV = p.dv;
    const float scale = p.scale;
    const bf16_t* __restrict__ gq = static_cast<const bf16_t*>(p.q);
    const bf16_t* __restrict__ gk = static_cast<const bf16_t*>(p.k);
    const bf16_t* __restrict__ gv = static_cast<const bf16_t*>(p.v);
    const bf16_t* __restrict__ gdo = static_cast<const bf16_t*>(bp.dout);
    const float* __restrict__ ga = static_cast<const float*>(p.alpha);
    const float* __restrict__ gb = p.beta;

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, ln = l & 15, lg = l >> 4;
    const int c = tid % DVT, rg = tid / DVT, r0 = rg * RPT;
    const int nt = min(CH, len - ch * CH);
    const GradOut go = grad_out(bp, col0 / DVT);
    float* snap = lds;                                     // [CH / SNAP][DK][DVT]
    float* red = lds + (size_t)(CH / SNAP) * DK * DVT;     // [2][4 waves][DVT][2]
    int par = 0;

    // C-layout dS -> this thread's rows (through the first snapshot's space)
    __syncthreads();  // every wave is past its reads of this chunk's LDS
#pragma unroll
    for (int i = 0; i < STW; ++i) {
        const int st = w + 4 * i;
        if (st < NST) {
            const int ct = st / NJT, jj = st % NJT;
#pragma unroll
            for (int e = 0; e < 4; ++e) lds[(ct * 16 + lg * 4 + e) * DVT + jj * 16 + ln] = dS[i][e];
        }
    }
    __syncthreads();
    float G[RPT], S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) G[i] = lds[(r0 + i) * DVT + c];

    // sum of two per-column partials over the row groups (one barrier)
    auto rows_total = [&](float& x0, float& x1) {
        x0 += __shfl_xor(x0, 32, 64);
        x1 += __shfl_xor(x1, 32, 64);
        float* rb = red + (size_t)par * 4 * DVT * 2;
        if (l < 32) { rb[(w * DVT + c) * 2] = x0; rb[(w * DVT + c) * 2 + 1] = x1; }
        __syncthreads();
        x0 = (rb[c * 2] + rb[(DVT + c) * 2]) + (rb[(2 * DVT + c) * 2] + rb[(3 * DVT + c) * 2]);
        x1 = (rb[c * 2 + 1] + rb[(DVT + c) * 2 + 1]) + (rb[(2 * DVT + c) * 2 + 1] + rb[(3 * DVT + c) * 2 + 1]);
        par ^= 1;
    };
    // token t of the chunk, forward: S <- S~ + k u^T
    // (k and alpha are read again where used rather than held: they hit the
    // cache, and the path keeps few registers)
    auto fwd = [&](int t) {
        const size_t tok = (size_t)(t0 + (long)ch * CH + t) * H + h;
        float pv = 0.f, dummy = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const size_t e = tok * DK + r0 + i;
            S[i] *= ga[e];
            pv += to_f32(gk[e]) * S[i];
        }
        rows_total(pv, dummy);
        const float u = gb[tok] * (to_f32(gv[tok * DV + col0 + c]) - pv);
#pragma unroll
        for (int i = 0; i < RPT; ++i) S[i] += to_f32(gk[tok * DK + r0 + i]) * u;
    };
    auto load_state = [&](const float* src, int pitch) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) S[i] = src[(size_t)(r0 + i) * pitch + c];
    };
    auto save_snap = [&](int j) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) snap[((size_t)j * DK + r0 + i) * DVT + c] = S[i];
    };

    // snapshots of the state before tokens 0, 8, 16, .. of the chunk
    // (snapshot 0 overwrites the dS exchange, which every thread has read)
    const int nsnap = (nt + SNAP - 1) / SNAP;
    load_state(ckpt + col0, DV);
    __syncthreads();
    for (int j = 0; j < nsnap; ++j) {
        save_snap(j);
        if (j + 1 < nsnap)
            for (int t = j * SNAP; t < (j + 1) * SNAP; ++t) fwd(t);
    }

    for (int t = nt - 1; t >= 0; --t) {
        // the state before token t, from its snapshot
        const int j = t / SNAP;
        __syncthreads();  // snapshot writes (and the last token's reads) are done
        load_state(snap + (size_t)j * DK * DVT, DVT);
        for (int tt = j * SNAP; tt < t; ++tt) fwd(tt);

        const size_t tok = (size_t)(t0 + (long)ch * CH + t) * H + h;
        const float dov = to_f32(gdo[tok * DV + col0 + c]);
        const float beta = gb[tok];
        const float vv = to_f32(gv[tok * DV + col0 + c]);
        float pv = 0.f, pu = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const size_t e = tok * DK + r0 + i;
            const float kv = to_f32(gk[e]);
            G[i] += scale * to_f32(gq[e]) * dov;
            pv += kv * (ga[e] * S[i]);
            pu += kv * G[i];
        }
        rows_total(pv, pu);  // vh, du
        const float u = beta * (vv - pv);
        // per row: the three column sums (over the 32 lanes of a half wave),
        // added by one lane each
        for (int i = 0; i < RPT; ++i) {
            const size_t e = tok * DK + r0 + i;
            const float al = ga[e], kv = to_f32(gk[e]);
            const float st = al * S[i];                      // S~
            const float sn = st + kv * u;                    // the state after token t
            float gqv = scale * sn * dov;
            float gkv = G[i] * u - beta * st * pu;
            const float dst = G[i] - beta * kv * pu;         // dS~
            float gav = dst * S[i];
            G[i] = al * dst;
#pragma unroll
            for (int off = 1; off < 32; off *= 2) {
                gqv += __shfl_xor(gqv, off, 64);
                gkv += __shfl_xor(gkv, off, 64);
                gav += __shfl_xor(gav, off, 64);
            }
            if (c == 0) go.dq[e] = gqv;
            else if (c == 1) go.dk[e] = gkv;
            else if (c == 2) go.da[e] = gav;
        }
        if (rg == 0) {
            bp.dv[tok * DV + col0 + c] = beta * pu;
            float db = pu * (vv - pv);
#pragma unroll
            for (int off = 1; off < 32; off *= 2) db += __shfl_xor(db, off, 64);
            if (c == 0) go.db[tok] = db;
        }
    }

    // this thread's rows of dS -> C-layout tiles
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RPT; ++i) lds[(r0 + i) * DVT + c] = G[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < STW; ++i) {
        const int st = w + 4 * i;
        if (st < NST) {
            const int ct = st / NJT, jj = st % NJT;
#pragma unroll
            for (int e = 0; e < 4; ++e) dS[i][e] = lds[(ct * 16 + lg * 4 + e) * DVT + jj * 16 + ln];
        }
    }
    __syncthreads();  // the next chunk may overwrite this LDS
}

template <int DK, int DVT>
__global__ __launch_bounds__(BW_NTH, 1) void bwd_chunk_kernel(BwParams bp) {
    using Top = bf16_t;
    using L = BwLayout<DK, DVT>;
    using M = Mma<Top>;
    constexpr int CPT = DK / 64;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDV = L::LDV, LDD = L::LDD;
    constexpr int NJT = L::NJT, NST = L::NST, STW = L::STW;
    using R = BwRow<CPT>;
    const KParams& p = bp.base;
    static_assert((size_t)(8 * DK * DVT + 2 * 4 * DVT * 2) * 4 <= L::bytes, "token-chunk LDS");

    extern __shared__ __align__(16) unsigned char smem[];
    Top* sSPr = reinterpret_cast<Top*>(smem + L::oSPr);
    Top* sdWr = reinterpret_cast<Top*>(smem + L::odWr);
    Top* sdOr = reinterpret_cast<Top*>(smem + L::odOr);
    float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);
    float* sTot = reinterpret_cast<float*>(smem + L::oTot);
    float* sdlPn = reinterpret_cast<float*>(smem + L::odlPn);
    float* sDb1 = reinterpret_cast<float*>(smem + L::oDb1);
    float* sDb2 = reinterpret_cast<float*>(smem + L::oDb2);
    Top* sdOT = reinterpret_cast<Top*>(smem + L::odOT);
    Top* sLo = reinterpret_cast<Top*>(smem + L::oLo);
    float* sLd = reinterpret_cast<float*>(smem + L::oLd);
    Top* sMT = reinterpret_cast<Top*>(smem + L::oMT);
    Top* sYT = reinterpret_cast<Top*>(smem + L::oYT);
    Top* sUr = reinterpret_cast<Top*>(smem + L::oUr);
    Top* sdYr = reinterpret_cast<Top*>(smem + L::odYr);
    Top* sdXr = reinterpret_cast<Top*>(smem + L::odXr);
    Top* sdXT = reinterpret_cast<Top*>(smem + L::odXT);
    Top* sKr = reinterpret_cast<Top*>(smem + L::oKr);
    Top* sQr = reinterpret_cast<Top*>(smem + L::oQr);
    Top* sKc = reinterpret_cast<Top*>(smem + L::oKc);
    Top* sSPT = reinterpret_cast<Top*>(smem + L::oSPT);
    Top* sdWT = reinterpret_cast<Top*>(smem + L::odWT);
    Top* sTm = reinterpret_cast<Top*>(smem + L::oTm);
    Top* sTmT = reinterpret_cast<Top*>(smem + L::oTmT);
    Top* sDr = reinterpret_cast<Top*>(smem + L::oDr);
    Top* sDc = reinterpret_cast<Top*>(smem + L::oDc);
    Top* sdUT = reinterpret_cast<Top*>(smem + L::odUT);
    Top* sKrT = reinterpret_cast<Top*>(smem + L::oKrT);
    Top* sQrT = reinterpret_cast<Top*>(smem + L::oQrT);
    Top* sKcT = reinterpret_cast<Top*>(smem + L::oKcT);
    Top* sdA = reinterpret_cast<Top*>(smem + L::odA);
    Top* sdAT = reinterpret_cast<Top*>(smem + L::odAT);
    Top* sdM = reinterpret_cast<Top*>(smem + L::odM);
    Top* sdMT = reinterpret_cast<Top*>(smem + L::odMT);

    const WorkItem wi = decode_work(p);
    if (!wi.valid) return;
    const int H = p.H, h = wi.h, seq = wi.seq, jt = wi.jt, len = wi.len;
    const long t0 = wi.t0;
    const int DV = p.dv;
    const float scale = p.scale;
    const bf16_t* __restrict__ gq = static_cast<const bf16_t*>(p.q);
    const bf16_t* __restrict__ gk = static_cast<const bf16_t*>(p.k);
    const bf16_t* __restrict__ gv = static_cast<const bf16_t*>(p.v);
    const bf16_t* __restrict__ gdo = static_cast<const bf16_t*>(bp.dout);
    const float* __restrict__ ga = static_cast<const float*>(p.alpha);
    const float* __restrict__ gb = p.beta;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int ln = l & 15;
    const int lg = l >> 4;
    const int col0 = jt * DVT;
    const int c0 = l * CPT;
    const size_t sbase = ((size_t)seq * H + h) * DK * DV;
    const long slot0 = t0 / CH + 2 * (long)seq;
    const GradOut gout = grad_out(bp, jt);
    auto ckpt_at = [&](int ch) {
        return bp.ckpt + ((size_t)(slot0 + ch) * H + h) * DK * DV;
    };

    // ---- gradient of the chunk-end state, C-layout tiles w, w+4, ... ----
    f32x4 dS[STW];
#pragma unroll
    for (int i = 0; i < STW; ++i) {
        const int st = w + 4 * i;
        dS[i] = zero4();
        if (st < NST && bp.dsT) {
            const int ct = st / NJT, jj = st % NJT;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dS[i][e] = bp.dsT[sbase + (size_t)(ct * 16 + lg * 4 + e) * DV + col0 + jj * 16 + ln];
        }
    }

    // ---- register prefetch (row block w, channels c0..; v and dO in C-layout) ----
    typename R::B pq[16], pk[16];
    typename R::F pa[16];
    float pbeta = 0.f;
    bf16_t pv[NJT][4], pdo[NJT][4];
    auto load_rows = [&](int ch) {
        const int base_r = ch * CH + w * 16;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = min(base_r + r, len - 1);
            const size_t off = ((size_t)(t0 + t) * H + h) * DK + c0;
            pq[r] = R::ldb(gq + off);
            pk[r] = R::ldb(gk + off);
            pa[r] = R::ldf(ga + off);
        }
        if (w == 0) pbeta = gb[(size_t)(t0 + min(ch * CH + l, len - 1)) * H + h];
    };
    auto load_vdo = [&](int ch) {
#pragma unroll
        for (int jb = 0; jb < NJT; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = min(ch * CH + w * 16 + lg * 4 + e, len - 1);
                const size_t off = ((size_t)(t0 + t) * H + h) * DV + col0 + jb * 16 + ln;
                pv[jb][e] = gv[off];
                pdo[jb][e] = gdo[off];
            }
    };

    const int nch = (len + CH - 1) / CH;
    // running product of alpha over the rows of block w, one row further
    auto step_run = [&](float (&run)[CPT], const typename R::F& af, int r, int nvalid) {
        float a[CPT];
        R::uf(af, a);
#pragma unroll
        for (int c = 0; c < CPT; ++c) run[c] *= (r < nvalid) ? a[c] : 1.f;
    };

    // The sweep takes the chunk form until a chunk fails the range check; that
    // chunk and every one before it then go through the token-by-token chain
    // rule after the loop.  (The chunk form holds all 512 registers of a lane;
    // the token path placed inside the loop would make it spill.)
    // Descriptor over rows ch*CH .. of a [token][H][width] float tensor at
    // head h, ending with the sequence's last row in the chunk: the stores
    // of the rows past it are dropped.
    auto chunk_rsrc = [&](float* base, int ch, int width) {
        const int nrow = min(len - ch * CH, CH);
        return make_rsrc(base + ((size_t)(t0 + (long)ch * CH) * H + h) * width, (uint32_t)(nrow * H * width * 4));
    };

    int token_from = -1;
    for (int ch = nch - 1; ch >= 0; --ch) {
        load_rows(ch);
        load_vdo(ch);
        // the chunk's start and end states, issued after the rows (phase 0 waits
        // for those only) and used in phase 1
        float s0v[STW][4], scv[STW][4];
        {
            const float* s0p = ckpt_at(ch);
            const float* scp = ckpt_at(ch + 1);
#pragma unroll
            for (int i = 0; i < STW; ++i) {
                const int st = w + 4 * i;
                const int ct = st / NJT, jj = st % NJT;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const size_t si = (size_t)(ct * 16 + lg * 4 + e) * DV + col0 + jj * 16 + ln;
                    s0v[i][e] = st < NST ? s0p[si] : 0.f;
                    scv[i][e] = st < NST ? scp[si] : 0.f;
                }
            }
        }
        // ================= phase 0: running products inside row block w ======
        typename R::B cq[16], ck[16];
        typename R::F ca[16];
        const int nvalid = len - (ch * CH + w * 16);
        {
            float run[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) run[c] = 1.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                cq[r] = pq[r]; ck[r] = pk[r]; ca[r] = pa[r];
                float a[CPT];
                R::uf(pa[r], a);
#pragma unroll
                for (int c = 0; c < CPT; ++c) run[c] *= (r < nvalid) ? a[c] : 1.f;
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) sTot[w * DK + c0 + c] = run[c];
            if (w == 0)
                sBeta[l] = (ch * CH + l < len) ? pbeta : 0.f;
        }
        __syncthreads();  // B1

        // Range check (every wave reads all channels' totals, so all waves
        // take the same branch).  The backward's bound is tighter than the
        // forward's: the gradient of the decays sums terms of every pair of
        // rows, and those of pairs on the same side of a token cancel in exact
        // arithmetic but leave bf16 rounding behind, which grows with the
        // decay across the chunk; below a half-chunk product of 2^-12 the
        // token-by-token path is the accurate one.
        {
            bool cbad = false;
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const float h1 = sTot[c0 + c] * sTot[DK + c0 + c];
                const float h2 = sTot[2 * DK + c0 + c] * sTot[3 * DK + c0 + c];
                cbad |= h1 < BW_DECAY_FLOOR || h2 < BW_DECAY_FLOOR;
            }
            if (__builtin_amdgcn_ballot_w64(cbad) != 0) {
                token_from = ch;
                break;
            }
        }

        // ================= phase 1: operands =================================
        // P_row / P_31 = (running product inside row block w) * fw with
        // fw = 1 / (t0 t1), 1 / t1, 1, t2 for w = 0..3 (t_b: row block b's product)
        float fw[CPT];
        {
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const float t0v = sTot[c0 + c], t1v = sTot[DK + c0 + c], t2v = sTot[2 * DK + c0 + c];
                fw[c] = (w == 0) ? fast_rcp(t0v * t1v) : (w == 1) ? fast_rcp(t1v) : (w == 2) ? 1.f : t2v;
            }
            float run[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) run[c] = 1.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = w * 16 + r;
                step_run(run, ca[r], r, nvalid);
                float kx[CPT], qx[CPT];
                R::ub(ck[r], kx);
                R::ub(cq[r], qx);
                Top kr[CPT], qr[CPT], kc[CPT];
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    const float kv = (r < nvalid) ? kx[c] : 0.f;
                    const float qv = (r < nvalid) ? qx[c] : 0.f;
                    const float ratio = run[c] * fw[c];
                    kr[c] = from_f32<Top>(kv * ratio);
                    qr[c] = from_f32<Top>(qv * ratio);
                    kc[c] = from_f32<Top>(kv * fast_rcp(ratio));
                }
                store_run<Top, CPT>(sKr + row * LDK + c0, kr);
                store_run<Top, CPT>(sQr + row * LDK + c0, qr);
                store_run<Top, CPT>(sKc + row * LDK + c0, kc);
            }
            // SP = Pm S0 (both layouts), dW = (Pn/Pm) dS (both layouts), and the
            // slice's part of rowsum(dS S_C) for the last row's decay
#pragma unroll
            for (int i = 0; i < STW; ++i) {
                const int st = w + 4 * i;
                if (st < NST) {
                    const int ct = st / NJT, jj = st % NJT;
                    f32x4 sp, dw;
                    float dl[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = ct * 16 + lg * 4 + e;
                        const float a0 = sTot[c], a1 = sTot[DK + c];
                        const float a2 = sTot[2 * DK + c], a3 = sTot[3 * DK + c];
                        const float pm = a0 * a1;
                        sp[e] = pm * s0v[i][e];
                        dw[e] = a2 * a3 * dS[i][e];
                        dl[e] = row16_total(dS[i][e] * scv[i][e]);
                    }
                    M::st4(sSPT + (jj * 16 + ln) * LDK + ct * 16 + lg * 4, sp);
                    M::st4(sdWT + (jj * 16 + ln) * LDK + ct * 16 + lg * 4, dw);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sSPr[(ct * 16 + lg * 4 + e) * LDV + jj * 16 + ln] = from_f32<Top>(sp[e]);
                        sdWr[(ct * 16 + lg * 4 + e) * LDV + jj * 16 + ln] = from_f32<Top>(dw[e]);
                        if (ln == 0) sdlPn[jj * DK + ct * 16 + lg * 4 + e] = dl[e];
                    }
                }
            }
            // dO of row block w in both layouts
#pragma unroll
            for (int jb = 0; jb < NJT; ++jb) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = (ch * CH + w * 16 + lg * 4 + e < len) ? to_f32(pdo[jb][e]) : 0.f;
                    sdOr[(w * 16 + lg * 4 + e) * LDV + jb * 16 + ln] = from_f32<Top>(x[e]);
                }
                M::st4(sdOT + (jb * 16 + ln) * LDC + w * 16 + lg * 4, x);
            }
        }
        __syncthreads();  // B2

        // ================= phase 2: Gram blocks, M^T, X, Y, Kc dW ==============
        f32x4 cA[3];   // A of this wave's Gram jobs, kept for dbeta
        f32x4 xr[NJT], du[NJT];
        {
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const int jn = w + 4 * q;
                cA[q] = zero4();
                if (jn < 10) {
                    const int a = (jn >= 6) ? 3 : (jn >= 3) ? 2 : (jn >= 1) ? 1 : 0;
                    const int b = jn - a * (a + 1) / 2;
                    f32x4 ca = zero4(), cm = zero4();
#pragma unroll
                    for (int s = 0; s < DK / 32; ++s) {
                        const auto fkc = M::ld32(sKc + (b * 16 + ln) * LDK + s * 32 + lg * 8);
                        const auto fkr = M::ld32(sKr + (a * 16 + ln) * LDK + s * 32 + lg * 8);
                        const auto fqr = M::ld32(sQr + (a * 16 + ln) * LDK + s * 32 + lg * 8);
                        ca = M::k32(fkc, fkr, ca);  // A[r = 16a + ln][i = 16b + 4lg + e]
                        cm = M::k32(fqr, fkc, cm);  // M[r = 16a + 4lg + e][i = 16b + ln]
                    }
                    const int r = a * 16 + ln;
                    const float br = sBeta[r];
                    if (a == b) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) ca[e] = (lg * 4 + e < ln) ? ca[e] : 0.f;
                        float4 ld = make_float4(br * ca[0], br * ca[1], br * ca[2], br * ca[3]);
                        *reinterpret_cast<float4*>(sLd + (a * 16 + ln) * L::LDL + lg * 4) = ld;
#pragma unroll
                        for (int e = 0; e < 4; ++e) cm[e] = (ln <= lg * 4 + e) ? cm[e] : 0.f;
                    } else {
                        f32x4 lo;
#pragma unroll
                        for (int e = 0; e < 4; ++e) lo[e] = br * ca[e];
                        M::st4(sLo + r * LDC + b * 16 + lg * 4, lo);
                        // the mirrored block of M^T (r-block < i-block) is zero
                        M::st4(sMT + (a * 16 + ln) * LDC + b * 16 + lg * 4, zero4());
                    }
                    cA[q] = ca;
                    // M^T[i = 16b + ln][r = 16a + 4lg + e]
                    M::st4(sMT + (b * 16 + ln) * LDC + a * 16 + lg * 4, cm);
                }
            }
            const int rowb = w * 16 + lg * 4;
#pragma unroll
            for (int jb = 0; jb < NJT; ++jb) {
                f32x4 cx = zero4(), cd = zero4();
#pragma unroll
                for (int s = 0; s < DK / 32; ++s) {
                    const auto fkr = M::ld32(sKr + (w * 16 + ln) * LDK + s * 32 + lg * 8);
                    const auto fkc = M::ld32(sKc + (w * 16 + ln) * LDK + s * 32 + lg * 8);
                    const auto fsp = M::ld32(sSPT + (jb * 16 + ln) * LDK + s * 32 + lg * 8);
                    const auto fdw = M::ld32(sdWT + (jb * 16 + ln) * LDK + s * 32 + lg * 8);
                    cx = M::k32(fkr, fsp, cx);
                    cd = M::k32(fkc, fdw, cd);
                }
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = ch * CH + rowb + e < len;
                    cx[e] = (ok ? to_f32(pv[jb][e]) : 0.f) - cx[e];
                    y[e] = sBeta[rowb + e] * cx[e];
                }
                xr[jb] = cx;
                du[jb] = cd;
                M::st4(sYT + (jb * 16 + ln) * LDC + rowb, y);
            }
        }
        __syncthreads();  // B3

        // ================= phase 3: T' = (I + Diag(beta) A)^{-1}; dU =========
        {
            // diagonal blocks: lane (block lg, column ln) solves L_aa x = e_ln, row by row
            float x[16];
            const float* La = sLd + lg * 16 * L::LDL;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == ln) ? 1.f : 0.f;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    if (q4 * 4 < r) {
                        const float4 v4 = *reinterpret_cast<const float4*>(La + r * L::LDL + q4 * 4);
                        const float lv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (q4 * 4 + u < r) acc -= lv[u] * x[q4 * 4 + u];
                    }
                }
                x[r] = acc;
            }
            Top* Dr = sDr + (size_t)w * 4 * 16 * LDD;
            Top* Dc = sDc + (size_t)w * 4 * 16 * LDD;
#pragma unroll
            for (int r = 0; r < 16; ++r) Dr[(lg * 16 + r) * LDD + ln] = from_f32<Top>(x[r]);
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 t4 = {x[r4 * 4], x[r4 * 4 + 1], x[r4 * 4 + 2], x[r4 * 4 + 3]};
                M::st4(Dc + (lg * 16 + ln) * LDD + r4 * 4, t4);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            // column block b = w of T': T'_bb = D_b, T'_ab = -D_a sum_{j=b}^{a-1} L_aj T'_jb
            const int b = w;
            f32x4 TB[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) TB[0][e] = to_f32(Dc[(b * 16 + ln) * LDD + lg * 4 + e]);
#pragma unroll
            for (int d = 1; d < 4; ++d) {
                const int a = b + d;
                if (a < 4) {
                    f32x4 y = zero4();
#pragma unroll
                    for (int jd = 0; jd < d; ++jd) {
                        const int j = b + jd;
                        const auto fa = M::ld16(sLo + (a * 16 + ln) * LDC + j * 16 + lg * 4);
                        y = M::k16(fa, M::pack16(TB[jd]), y);
                    }
                    const auto fd = M::ld16(Dr + (a * 16 + ln) * LDD + lg * 4);
                    f32x4 t = M::k16(fd, M::pack16(y), zero4());
                    TB[d][0] = -t[0]; TB[d][1] = -t[1]; TB[d][2] = -t[2]; TB[d][3] = -t[3];
                }
            }
            // TB[d] holds T'[16(b+d) + 4lg + e][16b + ln]; zero blocks elsewhere
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 t = (a >= b) ? TB[(a - b) & 3] : zero4();
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sTm[(a * 16 + lg * 4 + e) * LDC + b * 16 + ln] = from_f32<Top>(t[e]);
                M::st4(sTmT + (b * 16 + ln) * LDC + a * 16 + lg * 4, t);
            }
            // dU = Kc dW + scale M^T dO for rows i of block w
            const int s_lo = (w >= 2) ? 1 : 0;
#pragma unroll
            for (int jb = 0; jb < NJT; ++jb) {
                f32x4 cu = zero4();
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s >= s_lo) {
                        const auto fm = M::ld32(sMT + (w * 16 + ln) * LDC + s * 32 + lg * 8);
                        const auto fo = M::ld32(sdOT + (jb * 16 + ln) * LDC + s * 32 + lg * 8);
                        cu = M::k32(fm, fo, cu);
                    }
                }
                f32x4 d;
#pragma unroll
                for (int e = 0; e < 4; ++e) d[e] = du[jb][e] + scale * cu[e];
                M::st4(sdUT + (jb * 16 + ln) * LDC + w * 16 + lg * 4, d);
            }
        }
        __syncthreads();  // B4

        // ================= phase 4: U = T' Y, dY = T'^T dU, dX, dv ===========
        {
            const Rsrc rdv = chunk_rsrc(bp.dv, ch, DV);
            const int ns = (w >= 2) ? 2 : 1;
            const int s_lo = (w >= 2) ? 1 : 0;
            const int rowb = w * 16 + lg * 4;
            float db1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jb = 0; jb < NJT; ++jb) {
                f32x4 cu = zero4(), cy = zero4();
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s < ns) {
                        const auto ft = M::ld32(sTm + (w * 16 + ln) * LDC + s * 32 + lg * 8);
                        const auto fy = M::ld32(sYT + (jb * 16 + ln) * LDC + s * 32 + lg * 8);
                        cu = M::k32(ft, fy, cu);
                    }
                    if (s >= s_lo) {
                        const auto ft = M::ld32(sTmT + (w * 16 + ln) * LDC + s * 32 + lg * 8);
                        const auto fu = M::ld32(sdUT + (jb * 16 + ln) * LDC + s * 32 + lg * 8);
                        cy = M::k32(ft, fu, cy);
                    }
                }
                f32x4 dx;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = rowb + e;
                    dx[e] = sBeta[r] * cy[e];
                    db1[e] += cy[e] * xr[jb][e];
                    sUr[r * LDV + jb * 16 + ln] = from_f32<Top>(cu[e]);
                    sdYr[r * LDV + jb * 16 + ln] = from_f32<Top>(cy[e]);
                    sdXr[r * LDV + jb * 16 + ln] = from_f32<Top>(dx[e]);
                    // lane part: row rowb, column col0 + ln; wave part: row e, column tile jb
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dx[e]), rdv,
                                                          (uint32_t)((rowb * H * DV + col0 + ln) * 4),
                                                          (e * H * DV + jb * 16) * 4, 0);
                }
                M::st4(sdXT + (jb * 16 + ln) * LDC + rowb, dx);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float tot = row16_total(db1[e]);
                if (ln == 0) sDb1[rowb + e] = tot;
            }
        }
        __syncthreads();  // B5

        // ================= phase 5: G = dY U^T -> dA, dM; transposed operands =
        {
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const int jn = w + 4 * q;
                if (jn < 10) {
                    const int a = (jn >= 6) ? 3 : (jn >= 3) ? 2 : (jn >= 1) ? 1 : 0;
                    const int b = jn - a * (a + 1) / 2;
                    f32x4 cg = zero4(), cm = zero4();
#pragma unroll
                    for (int s = 0; s < DVT / 32; ++s) {
                        const auto fu = M::ld32(sUr + (b * 16 + ln) * LDV + s * 32 + lg * 8);
                        const auto fy = M::ld32(sdYr + (a * 16 + ln) * LDV + s * 32 + lg * 8);
                        const auto fo = M::ld32(sdOr + (a * 16 + ln) * LDV + s * 32 + lg * 8);
                        cg = M::k32(fu, fy, cg);  // G[r = 16a + ln][i = 16b + 4lg + e]
                        cm = M::k32(fu, fo, cm);  // (dO U^T)[r][i]
                    }
                    if constexpr (DVT % 32 != 0) {
                        const auto fu = M::ld16(sUr + (b * 16 + ln) * LDV + (DVT / 32) * 32 + lg * 4);
                        const auto fy = M::ld16(sdYr + (a * 16 + ln) * LDV + (DVT / 32) * 32 + lg * 4);
                        const auto fo = M::ld16(sdOr + (a * 16 + ln) * LDV + (DVT / 32) * 32 + lg * 4);
                        cg = M::k16(fu, fy, cg);
                        cm = M::k16(fu, fo, cm);
                    }
                    const int r = a * 16 + ln;
                    const float br = sBeta[r];
                    f32x4 da, dm;
                    float db2 = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int il = lg * 4 + e;
                        const bool strict = (a > b) || (il < ln);
                        const bool lower = (a > b) || (il <= ln);
                        da[e] = strict ? -br * cg[e] : 0.f;
                        dm[e] = lower ? scale * cm[e] : 0.f;
                        db2 += strict ? cg[e] * cA[q][e] : 0.f;
                    }
                    db2 += __shfl_xor(db2, 16, 64);
                    db2 += __shfl_xor(db2, 32, 64);
                    if (lg == 0) sDb2[jn * 16 + ln] = db2;
                    M::st4(sdA + r * LDC + b * 16 + lg * 4, da);
                    M::st4(sdM + r * LDC + b * 16 + lg * 4, dm);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sdAT[(b * 16 + lg * 4 + e) * LDC + r] = from_f32<Top>(da[e]);
                        sdMT[(b * 16 + lg * 4 + e) * LDC + r] = from_f32<Top>(dm[e]);
                    }
                    if (a != b) {  // the mirrored blocks above the diagonal are zero
                        M::st4(sdA + (b * 16 + ln) * LDC + a * 16 + lg * 4, zero4());
                        M::st4(sdM + (b * 16 + ln) * LDC + a * 16 + lg * 4, zero4());
                        M::st4(sdAT + (a * 16 + ln) * LDC + b * 16 + lg * 4, zero4());
                        M::st4(sdMT + (a * 16 + ln) * LDC + b * 16 + lg * 4, zero4());
                    }
                }
            }
            // transposed operands Kr^T, Qr^T, Kc^T of row block w (16-token runs)
            Top krt[CPT][16], qrt[CPT][16], kct[CPT][16];
            float run[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) run[c] = 1.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                step_run(run, ca[r], r, nvalid);
                float kx[CPT], qx[CPT];
                R::ub(ck[r], kx);
                R::ub(cq[r], qx);
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    const float kv = (r < nvalid) ? kx[c] : 0.f;
                    const float qv = (r < nvalid) ? qx[c] : 0.f;
                    const float ratio = run[c] * fw[c];
                    krt[c][r] = from_f32<Top>(kv * ratio);
                    qrt[c][r] = from_f32<Top>(qv * ratio);
                    kct[c][r] = from_f32<Top>(kv * fast_rcp(ratio));
                }
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                store_run<Top, 16>(sKrT + (c0 + c) * LDC + w * 16, krt[c]);
                store_run<Top, 16>(sQrT + (c0 + c) * LDC + w * 16, qrt[c]);
                store_run<Top, 16>(sKcT + (c0 + c) * LDC + w * 16, kct[c]);
            }
        }
        __syncthreads();  // B6

        // ================= phase 6: the chain dS; dq, dk and dlogP per tile ====
        // C-layout: lane (lg, ln) of wave w holds rows 16w + 4lg + e (e = 0..3)
        // of channel 16 ct + ln.  The per-element decay factors are formed here
        // from alpha reloaded in this layout (prefix products inside the lane's
        // four rows, then across the four lane groups).
        const Rsrc rdq = chunk_rsrc(gout.dq, ch, DK), rdk = chunk_rsrc(gout.dk, ch, DK);
        float dls[DK / 16][4];  // suffix sums of dlogP inside row block w
        {
#pragma unroll
            for (int i = 0; i < STW; ++i) {
                const int st = w + 4 * i;
                if (st < NST) {
                    const int ct = st / NJT, jj = st % NJT;
                    f32x4 cq = zero4(), ck = zero4();
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const auto fq = M::ld32(sQrT + (ct * 16 + ln) * LDC + s * 32 + lg * 8);
                        const auto fo = M::ld32(sdOT + (jj * 16 + ln) * LDC + s * 32 + lg * 8);
                        const auto fk = M::ld32(sKrT + (ct * 16 + ln) * LDC + s * 32 + lg * 8);
                        const auto fx = M::ld32(sdXT + (jj * 16 + ln) * LDC + s * 32 + lg * 8);
                        cq = M::k32(fq, fo, cq);
                        ck = M::k32(fk, fx, ck);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = ct * 16 + lg * 4 + e;
                        const float pm = sTot[c] * sTot[DK + c];
                        const float pn = pm * sTot[2 * DK + c] * sTot[3 * DK + c];
                        dS[i][e] = pn * dS[i][e] + pm * (scale * cq[e] - ck[e]);
                    }
                }
            }
            const int rowb = w * 16 + lg * 4;
            // alpha, k and q of an element block in this layout (L2-resident: loaded in
            // phase 0), read one block ahead of their use
            float na[4], nk[4], nq[4];
            auto ld_block = [&](int ct) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = min(ch * CH + rowb + e, len - 1);
                    const size_t off = ((size_t)(t0 + t) * H + h) * DK + ct * 16 + ln;
                    na[e] = ga[off];
                    nk[e] = to_f32(gk[off]);
                    nq[e] = to_f32(gq[off]);
                }
            };
            ld_block(0);
#pragma unroll
            for (int ct = 0; ct < DK / 16; ++ct) {
                const int c = ct * 16 + ln;
                float ae[4], ke[4], qe[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = ch * CH + rowb + e < len;
                    ae[e] = ok ? na[e] : 1.f;
                    ke[e] = ok ? nk[e] : 0.f;
                    qe[e] = ok ? nq[e] : 0.f;
                }
                if (ct + 1 < DK / 16) ld_block(ct + 1);
                f32x4 aq = zero4(), ak = zero4(), ac = zero4(), aqo = zero4(), akx = zero4();
                // contractions over the slice's value columns
#pragma unroll
                for (int s = 0; s < DVT / 32; ++s) {
                    const auto fo = M::ld32(sdOr + (w * 16 + ln) * LDV + s * 32 + lg * 8);
                    const auto fx = M::ld32(sdXr + (w * 16 + ln) * LDV + s * 32 + lg * 8);
                    const auto fu = M::ld32(sUr + (w * 16 + ln) * LDV + s * 32 + lg * 8);
                    const auto fsp = M::ld32(sSPr + (ct * 16 + ln) * LDV + s * 32 + lg * 8);
                    const auto fdw = M::ld32(sdWr + (ct * 16 + ln) * LDV + s * 32 + lg * 8);
                    aqo = M::k32(fo, fsp, aqo);   // dO SP^T
                    akx = M::k32(fx, fsp, akx);   // dX SP^T
                    ac = M::k32(fu, fdw, ac);     // U dW^T
                }
                if constexpr (DVT % 32 != 0) {
                    constexpr int sv = (DVT / 32) * 32;
                    const auto fo = M::ld16(sdOr + (w * 16 + ln) * LDV + sv + lg * 4);
                    const auto fx = M::ld16(sdXr + (w * 16 + ln) * LDV + sv + lg * 4);
                    const auto fu = M::ld16(sUr + (w * 16 + ln) * LDV + sv + lg * 4);
                    const auto fsp = M::ld16(sSPr + (ct * 16 + ln) * LDV + sv + lg * 4);
                    const auto fdw = M::ld16(sdWr + (ct * 16 + ln) * LDV + sv + lg * 4);
                    aqo = M::k16(fo, fsp, aqo);
                    akx = M::k16(fx, fsp, akx);
                    ac = M::k16(fu, fdw, ac);
                }
                // contractions over the chunk's tokens
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const auto fdm = M::ld32(sdM + (w * 16 + ln) * LDC + s * 32 + lg * 8);
                    const auto fda = M::ld32(sdA + (w * 16 + ln) * LDC + s * 32 + lg * 8);
                    const auto fdat = M::ld32(sdAT + (w * 16 + ln) * LDC + s * 32 + lg * 8);
                    const auto fdmt = M::ld32(sdMT + (w * 16 + ln) * LDC + s * 32 + lg * 8);
                    const auto fkc = M::ld32(sKcT + (ct * 16 + ln) * LDC + s * 32 + lg * 8);
                    const auto fkr = M::ld32(sKrT + (ct * 16 + ln) * LDC + s * 32 + lg * 8);
                    const auto fqr = M::ld32(sQrT + (ct * 16 + ln) * LDC + s * 32 + lg * 8);
                    aq = M::k32(fdm, fkc, aq);     // dM Kc
                    ak = M::k32(fda, fkc, ak);     // dA Kc
                    ac = M::k32(fdat, fkr, ac);    // dA^T Kr
                    ac = M::k32(fdmt, fqr, ac);    // dM^T Qr
                }
                // P_r / Pm for the lane's four rows: prefix inside the lane, then
                // the products of the earlier lane groups, the row block's factor
                float pre4[4];
                float run = 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) { run *= ae[e]; pre4[e] = run; }
                // exclusive product over lane groups lg' < lg (lanes ln + 16 lg')
                float g1 = __shfl_up(run, 16, 64);
                float excl = (lg >= 1) ? g1 : 1.f;
                float g2 = __shfl_up(run * excl, 32, 64);  // groups lg-2, lg-3 combined
                excl = (lg >= 2) ? excl * g2 : excl;
                // the factor of row block w: 1 / (t0 t1), 1 / t1, 1, t2
                const float fwc = (w == 0) ? fast_rcp(sTot[c] * sTot[DK + c])
                                : (w == 1) ? fast_rcp(sTot[DK + c]) : (w == 2) ? 1.f : sTot[2 * DK + c];
                float dl[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ratio = fwc * excl * pre4[e];  // P_r / Pm
                    const float irat = fast_rcp(ratio);
                    const float gq = scale * aqo[e] + aq[e];
                    const float gkr = ak[e] - akx[e];
                    const float gkc = ac[e];
                    // (non-temporal: the planes are read once, by the last pass)
                    // lane part: row rowb, channel ln; wave part: row e, channel tile ct
                    const uint32_t lo = (uint32_t)((rowb * H * DK + ln) * 4);
                    const int so = (e * H * DK + ct * 16) * 4;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gq * ratio), rdq, lo, so, CPOL_NT);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gkr * ratio + gkc * irat), rdk, lo, so,
                                                          CPOL_NT);
                    dl[e] = (gkr * ke[e] + gq * qe[e]) * ratio - gkc * ke[e] * irat;
                }
                if (w == 3 && lg == 3) {  // the last row also carries the chunk-end decay
                    dl[3] += sdlPn[c];
                    if (NJT > 1) dl[3] += sdlPn[DK + c];
                }
                // suffix sums over the block's rows: inside the lane, then across groups
                float suf = 0.f;
#pragma unroll
                for (int e = 3; e >= 0; --e) { suf += dl[e]; dl[e] = suf; }
                // exclusive suffix over lane groups lg' > lg
                const float h1 = __shfl_down(suf, 16, 64);
                float later = (lg <= 2) ? h1 : 0.f;
                const float h2 = __shfl_down(suf + later, 32, 64);
                later = (lg <= 1) ? later + h2 : later;
#pragma unroll
                for (int e = 0; e < 4; ++e) dls[ct][e] = dl[e] + later;
            }
        }
        __syncthreads();  // B7: everyone is done reading sTot
        // ================= phase 7: dalpha (suffix across row blocks), dbeta ==
        {
            const Rsrc rda = chunk_rsrc(gout.da, ch, DK), rdb = chunk_rsrc(gout.db, ch, 1);
            const int rowb = w * 16 + lg * 4;
            // alpha of the lane's elements, read before the barrier below
            float av[DK / 16][4];
#pragma unroll
            for (int ct = 0; ct < DK / 16; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = min(ch * CH + rowb + e, len - 1);
                    av[ct][e] = ga[((size_t)(t0 + t) * H + h) * DK + ct * 16 + ln];
                }
            if (lg == 0) {  // block totals: the suffix at the block's first row
#pragma unroll
                for (int ct = 0; ct < DK / 16; ++ct) sTot[w * DK + ct * 16 + ln] = dls[ct][0];
            }
            __syncthreads();  // B8
#pragma unroll
            for (int ct = 0; ct < DK / 16; ++ct) {
                const int c = ct * 16 + ln;
                float later = 0.f;
                for (int b = w + 1; b < 4; ++b) later += sTot[b * DK + c];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((dls[ct][e] + later) / av[ct][e]), rda,
                                                          (uint32_t)((rowb * H * DK + ln) * 4),
                                                          (e * H * DK + ct * 16) * 4, CPOL_NT);
            }
            if (w == 0) {
                const int r = l;
                // jobs (a, b) of row block a = r / 16, in a fixed order
                const int a = r >> 4;
                float db = sDb1[r];
                for (int b = 0; b <= a; ++b) db -= sDb2[(a * (a + 1) / 2 + b) * 16 + (r & 15)];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(db), rdb, (uint32_t)(r * H * 4), 0, 0);
            }
        }
        __syncthreads();  // B9: LDS reuse by the next chunk
    }
    for (int ch = token_from; ch >= 0; --ch)
        bw_token_chunk<DK, DVT, STW>(bp, seq, h, t0, len, ch, col0, ckpt_at(ch), dS,
                                     reinterpret_cast<float*>(smem));

    // ---- the initial state's gradient: this slice's columns ----
#pragma unroll
    for (int i = 0; i < STW; ++i) {
        const int st = w + 4 * i;
        if (st < NST) {
            const int ct = st / NJT, jj = st % NJT;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bp.ds0[sbase + (size_t)(ct * 16 + lg * 4 + e) * DV + col0 + jj * 16 + ln] = dS[i][e];
        }
    }
}

// out[i] = ((out[i] + p_1[i]) + p_2[i]) + ..., with p_j = part + (j - 1) * stride:
// the slices' partial sums added in a fixed order, four elements per thread
// (n4 float4 groups; out, part and stride keep 16-byte alignment)
__global__ void bw_sum_planes_kernel(float* __restrict__ out, const float* __restrict__ part,
                                     size_t n4, size_t stride, int nparts) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
         i += (size_t)gridDim.x * blockDim.x) {
        float4 acc = reinterpret_cast<const float4*>(out)[i];
        for (int j = 0; j < nparts; ++j) {
            const float4 x = reinterpret_cast<const float4*>(part + (size_t)j * stride)[i];
            acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
        }
        reinterpret_cast<float4*>(out)[i] = acc;
    }
}
// the same for a length that need not be a multiple of four
__global__ void bw_sum_planes1_kernel(float* __restrict__ out, const float* __restrict__ part,
                                      size_t n, size_t stride, int nparts) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x) {
        float acc = out[i];
        for (int j = 0; j < nparts; ++j) acc += part[(size_t)j * stride + i];
        out[i] = acc;
    }
}

template <int DK>
hipError_t launch_bw(const BwParams& bp, hipStream_t stream) {
    constexpr int DVT = 32;
    using Lay = BwLayout<DK, DVT>;
    const int groups = (bp.base.units + 7) / 8;
    const long grid = 8L * bp.base.njt_all * groups;
    static const hipError_t attr = hipFuncSetAttribute(
        (const void*)bwd_chunk_kernel<DK, DVT>, hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((bwd_chunk_kernel<DK, DVT>), dim3((unsigned)grid), dim3(BW_NTH),
                       Lay::bytes, stream, bp);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t stream) {
    const int nseq = a.cu_seqlens ? a.num_seqs : a.B;
    const int units = nseq * a.H;
    if (units == 0) return hipSuccess;
    const long tokens = a.cu_seqlens ? a.T : (long)a.B * a.T;
    float* ckpt = static_cast<float*>(a.workspace);
    float* part = reinterpret_cast<float*>(static_cast<char*>(a.workspace) +
                                           bwd_chunk_ckpt_bytes(tokens, nseq, a.H, a.dk, a.dv));
    // 1. the forward with a checkpoint of the state at every chunk start
    ChunkArgs f;
    f.q = a.q; f.k = a.k; f.v = a.v; f.alpha = a.alpha; f.beta = a.beta;
    f.s0 = a.s0; f.o = nullptr; f.sT = nullptr;
    f.B = a.B; f.T = a.T; f.H = a.H; f.dk = a.dk; f.dv = a.dv;
    f.bf16 = true;
    f.gate = 0;
    f.fuse = 0;
    f.cu_seqlens = a.cu_seqlens;
    f.num_seqs = a.num_seqs;
    f.order = nullptr;
    f.scale = a.scale;
    f.dvt = 0;
    f.generic = false;
    f.ckpt = ckpt;
    hipError_t e = launch_chunk_fwd(f, stream);
    if (e != hipSuccess) return e;
    // 2. the reverse sweep; every slice writes each of its gradient elements once
    const size_t nk = (size_t)tokens * a.H * a.dk, nb = bwd_chunk_beta_rows(tokens, a.H);
    BwParams bp;
    KParams& p = bp.base;
    p.q = a.q; p.k = a.k; p.v = a.v; p.alpha = a.alpha; p.beta = a.beta; p.s0 = a.s0;
    p.o = nullptr; p.sT = nullptr; p.cu_seqlens = a.cu_seqlens; p.order = nullptr;
    p.B = a.B; p.T = a.T; p.H = a.H; p.dv = a.dv;
    p.units = units;
    p.njt_all = a.dv / 32;
    p.gate = 0; p.fuse = 0;
    p.scale = a.scale;
    bp.dout = a.dout; bp.ckpt = ckpt; bp.dsT = a.dsT;
    bp.dq = a.g_q; bp.dk = a.g_k; bp.dv = a.g_v; bp.dalpha = a.g_alpha; bp.dbeta = a.g_beta;
    bp.ds0 = a.g_s0;
    bp.part = part; bp.nk = nk; bp.nb = nb;
    e = a.dk == 128 ? launch_bw<128>(bp, stream) : launch_bw<64>(bp, stream);
    if (e != hipSuccess || tokens == 0) return e;
    // 3. the slices' sums, in slice order
    const int nparts = a.dv / 32 - 1;
    const size_t stride = 3 * nk + nb;
    const unsigned g4 = (unsigned)std::min<size_t>((nk / 4 + 255) / 256, 8192);
    float* outs[] = {a.g_q, a.g_k, a.g_alpha};
    for (int i = 0; i < 3; ++i) {
        if (reinterpret_cast<uintptr_t>(outs[i]) % 16 == 0)
            hipLaunchKernelGGL(bw_sum_planes_kernel, dim3(g4), dim3(256), 0, stream, outs[i],
                               part + i * nk, nk / 4, stride, nparts);
        else  // an output at an odd offset: element by element
            hipLaunchKernelGGL(bw_sum_planes1_kernel, dim3(4 * g4), dim3(256), 0, stream, outs[i],
                               part + i * nk, nk, stride, nparts);
    }
    const size_t ntb = (size_t)tokens * a.H;
    hipLaunchKernelGGL(bw_sum_planes1_kernel, dim3((unsigned)std::min<size_t>((ntb + 255) / 256, 4096)),
                       dim3(256), 0, stream, a.g_beta, part + 3 * nk, ntb, stride, nparts);
    return hipGetLastError();
}

}  // namespace kda
