// chunk_fwd_bf16.hip -- the chunk-wise KDA forward for bf16 q/k/v on gfx950,
// organised as a two-stage pipeline inside each workgroup.
//
// Chunk algebra (derived from the update equation of "Kimi Delta Attention",
// section "KDA 的更新式"; the chunk-wise mode of bugfactory.tech news 3610,
// fifth paragraph).  For a 64-token chunk with start state S0, P_r the running
// product of alpha over the chunk's tokens 0..r (per key channel), Pm = P_31,
// Pn = P_63:
//     Kr = K*P/Pm, Qr = Q*P/Pm, Kc = K*Pm/P
//     A = tril_-1(Kr Kc^T) (rows scaled by beta: L = Diag(beta) A), M = tril(Qr Kc^T)
//     X = V - Kr (Pm*S0),   U = (I + L)^{-1} Diag(beta) X
//     O = scale (Qr (Pm*S0) + M U),   S <- Pn*S0 + (Pn/Pm) * (Kc^T U)
// U is found by block forward substitution over 16-token blocks,
//     U_a = D_a (beta_a X_a - sum_{b<a} L_ab U_b),   D_a = (I + L_aa)^{-1},
// so the 64x64 inverse is never formed.
//
// Roles.  A workgroup owns one (unit, 16*NJT value columns).  Waves
// 0..NJT-1 are consumers: each keeps one 16-column slice of the fp32 state in
// matrix-core accumulators and runs the state chain of chunk c (X, the solve,
// O, the next state); its U never leaves registers except for one LDS copy.
// Waves NJT..NJT+3 are producers: they build chunk c+1's operands (decays,
// Kr, Qr, Kc, Kc^T) and its Gram blocks (L, M) while the consumers work on c.
// Everything a consumer reads from a producer is double-buffered by chunk
// parity except Kc^T, which the producers hold in registers and write at the
// start of the consumer's chunk.  Two workgroup barriers per chunk:
//   segment 1: consumers  - D_a for chunk c, Pm*S0, X and Qr (Pm*S0)
//              producers  - write Kc^T(c); operands of chunk c+1
//   segment 2: consumers  - solve, O, next state (chunk c)
//              producers  - Gram blocks of chunk c+1
#include "chunk_common.h"

namespace kda {

template <int DK, int DVT>
struct Lay3 {
    static constexpr int NJT = DVT / 16;       // consumer waves
    static constexpr int NW = NJT + 4;         // + 4 producer waves
    static constexpr int NTH = 64 * NW;
    static constexpr int LDK = DK + 8;         // bf16 pitch of [token][channel] tiles
    static constexpr int LDC = CH + 8;         // bf16 pitch of [*][token] tiles
    static constexpr int LDB = 16 + 8;         // bf16 pitch of packed 16x16 blocks
    static constexpr int LDL = 20;             // fp32 pitch of the diagonal blocks of L
    static constexpr int BLK = 16 * LDB;       // elements per packed block

    static constexpr size_t szTok = (size_t)CH * LDK * 2;
    // one parity buffer
    static constexpr size_t bKr = 0;
    static constexpr size_t bQr = bKr + szTok;
    static constexpr size_t bLo = bQr + szTok;                  // -L_ab, b < a: 6 blocks
    static constexpr size_t bM = bLo + (size_t)6 * BLK * 2;     // M_ab, b <= a: 10 blocks
    static constexpr size_t bVec = bM + (size_t)10 * BLK * 2;   // fp32 Pm, Pn, Pn/Pm [3][DK]
    static constexpr size_t bBeta = bVec + (size_t)3 * DK * 4;  // fp32 [64]
    static constexpr size_t szBuf = (bBeta + CH * 4 + 15) / 16 * 16;
    // single copies
    static constexpr size_t oKcT = 2 * szBuf;                   // [DK][LDC]
    static constexpr size_t oKc = oKcT + (size_t)DK * LDC * 2;  // [64][LDK], producers only
    static constexpr size_t oLd = oKc + szTok;                  // fp32 [4][16 cols][LDL]
    // consumer-private scratch
    static constexpr size_t cSP = 0;                            // [16][LDK] bf16: (Pm*S0)^T
    static constexpr size_t cU = cSP + (size_t)16 * LDK * 2;    // [16][LDC] bf16: U^T
    static constexpr size_t cD = cU + (size_t)16 * LDC * 2;     // 4 blocks: D_a row-major
    static constexpr size_t szC = (cD + (size_t)4 * BLK * 2 + 15) / 16 * 16;
    static constexpr size_t oCons = oLd + (size_t)4 * 16 * LDL * 4;
    static constexpr size_t bytes = oCons + NJT * szC;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    bf16x4 h;
    h[0] = (bf16_t)a; h[1] = (bf16_t)b; h[2] = (bf16_t)c; h[3] = (bf16_t)d;
    return __builtin_bit_cast(uint2, h);
}
__device__ __forceinline__ void unpack4(uint2 w, float* x) {
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
}
__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int DK, int DVT>
__global__ __launch_bounds__((Lay3<DK, DVT>::NTH), 1) void chunk_fwd_bf16_kernel(KParams p) {
    using L = Lay3<DK, DVT>;
    using Mf = Mma<bf16_t>;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDB = L::LDB, LDL = L::LDL, BLK = L::BLK;
    constexpr int NJT = L::NJT;
    constexpr int NCT = DK / 16;          // 16-row tiles of a state slice
    constexpr int CPW = DK / 4;           // channels per producer wave
    constexpr int CQW = CPW / 4;          // channel quads per producer wave (8 or 4)
    constexpr int RGW = 64 / CQW;         // row groups per producer wave (8 or 16)
    constexpr int RPT = CH / RGW;         // rows per producer lane (8 or 4)

    extern __shared__ __align__(16) unsigned char smem[];
    auto buf = [&](int par, size_t off) { return smem + par * L::szBuf + off; };
    bf16_t* sKcT = reinterpret_cast<bf16_t*>(smem + L::oKcT);
    bf16_t* sKc = reinterpret_cast<bf16_t*>(smem + L::oKc);
    float* sLd = reinterpret_cast<float*>(smem + L::oLd);

    const WorkItem wi = decode_work(p);
    if (!wi.valid) return;
    const int H = p.H, h = wi.h, jt = wi.jt, len = wi.len;
    const long t0 = wi.t0;
    const int DV = p.dv;
    const int nch = (len + CH - 1) / CH;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int ln = l & 15, lg = l >> 4;
    const bool consumer = w < NJT;

    // Values a wave carries from one chunk to the next live in one register
    // array shared by the two roles (a wave keeps its role for the whole
    // kernel), so the allocation is the larger of the two sets, not the sum.
    //   producer: q rows RF[0,2RPT) | k rows RF[16,16+2RPT) | alpha rows
    //             RF[32,32+4RPT) | Kc^T bf16 pairs RF[64,64+2RPT) | beta RF[80]
    //   consumer: state RF[0,4NCT) | beta-scaled X RF[32,48) | Qr(Pm S0) RF[48,64)
    //             | V bf16 pairs RF[64,72)
    constexpr int RFN = 81;
    uint32_t RF[RFN];
#pragma unroll
    for (int i = 0; i < RFN; ++i) RF[i] = 0u;
    auto rf_f = [&](int i) { return __uint_as_float(RF[i]); };
    auto rf_f4 = [&](int i) { f32x4 v = {rf_f(i), rf_f(i + 1), rf_f(i + 2), rf_f(i + 3)}; return v; };
    auto rf_set4 = [&](int i, f32x4 v) {
        RF[i] = __float_as_uint(v[0]); RF[i + 1] = __float_as_uint(v[1]);
        RF[i + 2] = __float_as_uint(v[2]); RF[i + 3] = __float_as_uint(v[3]);
    };

    // ------------------------------------------------------------ producers
    const int pw = w - NJT;                       // producer index 0..3
    const int cq = l % CQW, rg = l / CQW;
    const int pc0 = pw * CPW + cq * 4;            // channels pc0..pc0+3
    const int pr0 = rg * RPT;                     // rows pr0..pr0+RPT-1
    static_assert(2 * RPT <= 16 && 4 * RPT <= 32 && NCT * 4 <= 32, "register file layout");
    const bf16_t* __restrict__ gq = static_cast<const bf16_t*>(p.q);
    const bf16_t* __restrict__ gk = static_cast<const bf16_t*>(p.k);
    const float* __restrict__ ga = p.alpha;
    const float* __restrict__ gb = p.beta;

    auto p_load = [&](int ch) {  // raw rows of chunk ch; rows past the end re-read the last one
        // uniform base of the chunk's first token plus 32-bit lane offsets
        const size_t cbase = ((size_t)(t0 + (long)ch * CH) * H + h) * DK;
        const bf16_t* bq = gq + cbase;
        const bf16_t* bk = gk + cbase;
        const float* ba = ga + cbase;
        const int last = len - 1 - ch * CH;  // last valid row of this chunk
#pragma unroll
        for (int rr = 0; rr < RPT; ++rr) {
            const unsigned off = (unsigned)(min(pr0 + rr, last) * H * DK + pc0);
            const uint2 q2 = *reinterpret_cast<const uint2*>(bq + off);
            const uint2 k2 = *reinterpret_cast<const uint2*>(bk + off);
            const uint4 a4 = *reinterpret_cast<const uint4*>(ba + off);
            RF[2 * rr] = q2.x; RF[2 * rr + 1] = q2.y;
            RF[16 + 2 * rr] = k2.x; RF[16 + 2 * rr + 1] = k2.y;
            RF[32 + 4 * rr] = a4.x; RF[32 + 4 * rr + 1] = a4.y;
            RF[32 + 4 * rr + 2] = a4.z; RF[32 + 4 * rr + 3] = a4.w;
        }
        if (pw == 0) RF[80] = __float_as_uint(gb[(size_t)(t0 + (long)ch * CH) * H + h + (unsigned)(min(l, last) * H)]);
    };

    // decayed operands of chunk ch into parity buffer ch & 1 (Kc^T kept in RF)
    auto p_operands = [&](int ch) {
        const bool full = ch * CH + CH <= len;
        const int par = ch & 1;
        const int nval = len - (ch * CH + pr0);   // valid rows of this lane
        // alpha of row rr, channel c (1 past the end of the sequence)
        auto alpha_at = [&](int rr, int c) {
            return (full || rr < nval) ? rf_f(32 + 4 * rr + c) : 1.f;
        };
        float pr[RPT][4];  // running product inside the lane's rows, later P_r / Pm
        float incl[4], excl[4], pm[4], pn[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float run = alpha_at(0, c);
            pr[0][c] = run;
#pragma unroll
            for (int rr = 1; rr < RPT; ++rr) { run *= alpha_at(rr, c); pr[rr][c] = run; }
            incl[c] = run;
        }
        // inclusive product over the row groups 0..rg (same channels, lanes l - d*CQW)
#pragma unroll
        for (int d = 1; d < RGW; d *= 2) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float y = __shfl(incl[c], (l - d * CQW) & 63, 64);
                if (rg >= d) incl[c] *= y;
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float y = __shfl(incl[c], (l - CQW) & 63, 64);
            excl[c] = rg >= 1 ? y : 1.f;
            pm[c] = __shfl(incl[c], cq + (RGW / 2 - 1) * CQW, 64);  // through row 31
            pn[c] = __shfl(incl[c], cq + (RGW - 1) * CQW, 64);      // through row 63
        }
        float* vec = reinterpret_cast<float*>(buf(par, L::bVec));
        if (rg == 0) {
            float ipm[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) ipm[c] = fast_rcp(pm[c]);
            *reinterpret_cast<float4*>(vec + pc0) = make_float4(pm[0], pm[1], pm[2], pm[3]);
            *reinterpret_cast<float4*>(vec + DK + pc0) = make_float4(pn[0], pn[1], pn[2], pn[3]);
            *reinterpret_cast<float4*>(vec + 2 * DK + pc0) =
                make_float4(pn[0] * ipm[0], pn[1] * ipm[1], pn[2] * ipm[2], pn[3] * ipm[3]);
        }
        if (pw == 0) {
            float* beta = reinterpret_cast<float*>(buf(par, L::bBeta));
            beta[l] = (ch * CH + l < len) ? rf_f(80) : 0.f;
        }
        // pr becomes ratio_r = P_r / Pm;  g_r = Pm / P_r from a reverse running product
        float g[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float f = excl[c] * fast_rcp(pm[c]);
#pragma unroll
            for (int rr = 0; rr < RPT; ++rr) pr[rr][c] *= f;
            g[c] = fast_rcp(pr[RPT - 1][c]);
        }
        bf16_t* kr_b = reinterpret_cast<bf16_t*>(buf(par, L::bKr));
        bf16_t* qr_b = reinterpret_cast<bf16_t*>(buf(par, L::bQr));
        float kcp[4];  // Kc of the odd row of the current pair
#pragma unroll
        for (int rr = RPT - 1; rr >= 0; --rr) {
            float kx[4], qx[4];
            unpack4(make_uint2(RF[16 + 2 * rr], RF[16 + 2 * rr + 1]), kx);
            unpack4(make_uint2(RF[2 * rr], RF[2 * rr + 1]), qx);
            if (!full && rr >= nval) {
#pragma unroll
                for (int c = 0; c < 4; ++c) { kx[c] = 0.f; qx[c] = 0.f; }
            }
            float kr[4], qr[4], kc[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                kr[c] = kx[c] * pr[rr][c];
                qr[c] = qx[c] * pr[rr][c];
                kc[c] = kx[c] * g[c];
                if (rr > 0) g[c] *= alpha_at(rr, c);  // Pm / P_{rr-1} = (Pm / P_rr) * alpha_rr
                if (rr & 1) {
                    kcp[c] = kc[c];
                } else {  // Kc^T of this lane: channel c, rows (rr, rr+1) as one bf16 pair
                    bf16x2v pr2;
                    pr2[0] = (bf16_t)kc[c];
                    pr2[1] = (bf16_t)kcp[c];
                    RF[64 + c * (RPT / 2) + rr / 2] = __builtin_bit_cast(uint32_t, pr2);
                }
            }
            const int row = pr0 + rr;
            *reinterpret_cast<uint2*>(kr_b + row * LDK + pc0) = pack4(kr[0], kr[1], kr[2], kr[3]);
            *reinterpret_cast<uint2*>(qr_b + row * LDK + pc0) = pack4(qr[0], qr[1], qr[2], qr[3]);
            *reinterpret_cast<uint2*>(sKc + row * LDK + pc0) = pack4(kc[0], kc[1], kc[2], kc[3]);
        }
    };

    // Pull the raw rows of chunk ch into L2 ahead of their real load: every
    // producer lane touches two of the chunk's 128-byte lines (q, k or alpha).
    // The loaded words are folded into `pf_sink` one iteration later, when they
    // have long arrived, so the prefetch never holds up a wait.
    uint32_t pf[2] = {0u, 0u}, pf_sink = 0u;
    auto p_prefetch = [&](int ch) {
        const size_t cbase = ((size_t)(t0 + (long)ch * CH) * H + h) * DK;
        const int last = len - 1 - ch * CH;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int line = 2 * (pw * 64 + l) + i;      // 0..511: 8 lines per token row
            const int row = min(line >> 3, last), sub = line & 7;
            const unsigned roff = (unsigned)(row * H * DK);
            const uint32_t* src =
                sub < 2 ? reinterpret_cast<const uint32_t*>(gq + cbase + roff) + sub * 32
              : sub < 4 ? reinterpret_cast<const uint32_t*>(gk + cbase + roff) + (sub - 2) * 32
                        : reinterpret_cast<const uint32_t*>(ga + cbase + roff) + (sub - 4) * 32;
            pf[i] = *src;
        }
    };

    auto p_write_kct = [&]() {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bf16_t* dst = sKcT + (pc0 + c) * LDC + pr0;
            if constexpr (RPT == 8) {
                *reinterpret_cast<uint4*>(dst) = make_uint4(RF[64 + c * 4], RF[64 + c * 4 + 1],
                                                            RF[64 + c * 4 + 2], RF[64 + c * 4 + 3]);
            } else {
                *reinterpret_cast<uint2*>(dst) = make_uint2(RF[64 + c * 2], RF[64 + c * 2 + 1]);
            }
        }
    };

    // Gram blocks of chunk ch: jobs (a, b), b <= a, dealt round-robin over the producers
    auto p_gram = [&](int ch) {
        const int par = ch & 1;
        const bf16_t* kr_b = reinterpret_cast<const bf16_t*>(buf(par, L::bKr));
        const bf16_t* qr_b = reinterpret_cast<const bf16_t*>(buf(par, L::bQr));
        bf16_t* lo_b = reinterpret_cast<bf16_t*>(buf(par, L::bLo));
        bf16_t* m_b = reinterpret_cast<bf16_t*>(buf(par, L::bM));
        const float* beta = reinterpret_cast<const float*>(buf(par, L::bBeta));
#pragma unroll
        for (int rep = 0; rep < 3; ++rep) {
            const int jn = pw + 4 * rep;
            if (jn < 10) {
                const int a = (jn >= 6) ? 3 : (jn >= 3) ? 2 : (jn >= 1) ? 1 : 0;
                const int b = jn - a * (a + 1) / 2;
                f32x4 cA = zero4(), cM = zero4();
#pragma unroll
                for (int s = 0; s < DK / 32; ++s) {
                    const auto fa = Mf::ld32(sKc + (b * 16 + ln) * LDK + s * 32 + lg * 8);
                    const auto fk = Mf::ld32(kr_b + (a * 16 + ln) * LDK + s * 32 + lg * 8);
                    const auto fq = Mf::ld32(qr_b + (a * 16 + ln) * LDK + s * 32 + lg * 8);
                    cA = Mf::k32(fa, fk, cA);
                    cM = Mf::k32(fa, fq, cM);
                }
                // lane holds A[r = 16a + ln][i = 16b + 4lg + e] (and M likewise)
                const float br = beta[a * 16 + ln];
                if (a == b) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = lg * 4 + e;  // L_aa stored column-major, fp32
                        sLd[(a * 16 + i) * LDL + ln] = (i < ln) ? br * cA[e] : 0.f;
                    }
                    f32x4 mm;
#pragma unroll
                    for (int e = 0; e < 4; ++e) mm[e] = (lg * 4 + e <= ln) ? cM[e] : 0.f;
                    Mf::st4(m_b + jn * BLK + ln * LDB + lg * 4, mm);
                } else {
                    f32x4 lo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) lo[e] = -br * cA[e];
                    Mf::st4(lo_b + (a * (a - 1) / 2 + b) * BLK + ln * LDB + lg * 4, lo);
                    Mf::st4(m_b + jn * BLK + ln * LDB + lg * 4, cM);
                }
            }
        }
    };

    // ------------------------------------------------------------ consumers
    const int cj = w;                        // consumer column tile
    const int col = jt * DVT + cj * 16 + ln; // this lane's value column
    unsigned char* cbase = smem + L::oCons + (consumer ? cj : 0) * L::szC;
    bf16_t* cSP = reinterpret_cast<bf16_t*>(cbase + L::cSP);
    bf16_t* cU = reinterpret_cast<bf16_t*>(cbase + L::cU);
    bf16_t* cD = reinterpret_cast<bf16_t*>(cbase + L::cD);
    const bf16_t* __restrict__ gv = static_cast<const bf16_t*>(p.v);
    bf16_t* __restrict__ go = static_cast<bf16_t*>(p.o);
    const size_t sbase = ((size_t)wi.seq * H + h) * DK * DV;

    auto c_load_v = [&](int ch) {
        const bf16_t* bv = gv + ((size_t)(t0 + (long)ch * CH) * H + h) * DV;
        const int last = len - 1 - ch * CH;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const unsigned off = (unsigned)(min(a * 16 + lg * 4 + e, last) * H * DV + col);
                const uint32_t hv = *reinterpret_cast<const uint16_t*>(bv + off);
                uint32_t& slot = RF[64 + 2 * a + e / 2];  // V rows 16a + 4lg + e, bf16 pairs
                slot = (e & 1) ? ((slot & 0x0000ffffu) | (hv << 16)) : ((slot & 0xffff0000u) | hv);
            }
    };

    if (consumer) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            if (p.s0) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    RF[4 * ct + e] = __float_as_uint(p.s0[sbase + (size_t)(ct * 16 + lg * 4 + e) * DV + col]);
            }
        }
        if (nch > 0) c_load_v(0);
    } else if (nch > 0) {
        p_load(0);
        p_operands(0);
        if (nch > 1) p_load(1);
    }
    __syncthreads();
    if (!consumer && nch > 0) p_gram(0);
    __syncthreads();

    for (int ch = 0; ch < nch; ++ch) {
        const int par = ch & 1;
        const bool full = ch * CH + CH <= len;
        // ======================= segment 1 =======================
        if (consumer) {
            // D_a = (I + L_aa)^{-1}: lane (block lg, column ln), right-looking
            {
                float xs[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) xs[r] = (r == ln) ? 1.f : 0.f;
                const float* La = sLd + lg * 16 * LDL;
#pragma unroll
                for (int i = 0; i < 15; ++i) {
                    float colv[16];
#pragma unroll
                    for (int q4 = (i + 1) / 4; q4 < 4; ++q4) {
                        const float4 v = ld4(La + i * LDL + q4 * 4);
                        colv[q4 * 4] = v.x; colv[q4 * 4 + 1] = v.y; colv[q4 * 4 + 2] = v.z; colv[q4 * 4 + 3] = v.w;
                    }
#pragma unroll
                    for (int r = i + 1; r < 16; ++r) xs[r] -= colv[r] * xs[i];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) cD[lg * BLK + r * LDB + ln] = (bf16_t)xs[r];
            }
            // (Pm * S0)^T as the B operand of X and Qr (Pm*S0)
            const float* vec = reinterpret_cast<const float*>(buf(par, L::bVec));
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float4 pm = ld4(vec + ct * 16 + lg * 4);
                const f32x4 sv = rf_f4(4 * ct);
                f32x4 sp = {pm.x * sv[0], pm.y * sv[1], pm.z * sv[2], pm.w * sv[3]};
                Mf::st4(cSP + ln * LDK + ct * 16 + lg * 4, sp);
            }
            wave_sync_lds();
            const bf16_t* kr_b = reinterpret_cast<const bf16_t*>(buf(par, L::bKr));
            const bf16_t* qr_b = reinterpret_cast<const bf16_t*>(buf(par, L::bQr));
            const float* beta = reinterpret_cast<const float*>(buf(par, L::bBeta));
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4 cx = zero4(), co = zero4();
#pragma unroll
                for (int s = 0; s < DK / 32; ++s) {
                    const auto fs = Mf::ld32(cSP + ln * LDK + s * 32 + lg * 8);
                    const auto fk = Mf::ld32(kr_b + (a * 16 + ln) * LDK + s * 32 + lg * 8);
                    const auto fq = Mf::ld32(qr_b + (a * 16 + ln) * LDK + s * 32 + lg * 8);
                    cx = Mf::k32(fk, fs, cx);
                    co = Mf::k32(fq, fs, co);
                }
                const float4 b4 = ld4(beta + a * 16 + lg * 4);
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = full || ch * CH + a * 16 + lg * 4 + e < len;
                    const uint32_t pair = RF[64 + 2 * a + e / 2];
                    const uint32_t bits = (e & 1) ? (pair & 0xffff0000u) : (pair << 16);
                    const float vv = ok ? __uint_as_float(bits) : 0.f;
                    const float be = e == 0 ? b4.x : e == 1 ? b4.y : e == 2 ? b4.z : b4.w;
                    y[e] = be * (vv - cx[e]);  // beta_r (v_r - (Kr Pm S0)_r)
                }
                rf_set4(32 + 4 * a, y);
                rf_set4(48 + 4 * a, co);
            }
            if (ch + 1 < nch) c_load_v(ch + 1);
        } else {
            p_write_kct();  // Kc^T of chunk ch (its Kc came with the operands one chunk ago)
            pf_sink ^= pf[0] ^ pf[1];
            if (ch + 3 < nch) p_prefetch(ch + 3);
            if (ch + 1 < nch) {
                p_operands(ch + 1);
                if (ch + 2 < nch) p_load(ch + 2);
            }
        }
        __syncthreads();
        // ======================= segment 2 =======================
        if (consumer) {
            const bf16_t* lo_b = reinterpret_cast<const bf16_t*>(buf(par, L::bLo));
            const bf16_t* m_b = reinterpret_cast<const bf16_t*>(buf(par, L::bM));
            const float* vec = reinterpret_cast<const float*>(buf(par, L::bVec));
            // U_a = D_a (Y_a - sum_{b<a} L_ab U_b); lo_b holds -L_ab
            f32x4 U[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4 acc = rf_f4(32 + 4 * a);
#pragma unroll
                for (int b = 0; b < a; ++b) {
                    const auto fl = Mf::ld16(lo_b + (a * (a - 1) / 2 + b) * BLK + ln * LDB + lg * 4);
                    acc = Mf::k16(fl, Mf::pack16(U[b]), acc);
                }
                const auto fd = Mf::ld16(cD + a * BLK + ln * LDB + lg * 4);
                U[a] = Mf::k16(fd, Mf::pack16(acc), zero4());
                Mf::st4(cU + ln * LDC + a * 16 + lg * 4, U[a]);
            }
            wave_sync_lds();
            // O_a = scale (OI_a + sum_{b<=a} M_ab U_b), k-steps of 32 tokens
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4 co = rf_f4(48 + 4 * a);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s == 0 || a >= 2) {
                        const int b = 2 * s + (lg >> 1);  // block of this lane's 8 k-values
                        Mf::F32 fm;
                        if (b <= a)
                            fm = Mf::ld32(m_b + (a * (a + 1) / 2 + b) * BLK + ln * LDB + (lg & 1) * 8);
                        else
                            fm.v = bf16x8{};
                        const auto fu = Mf::ld32(cU + ln * LDC + s * 32 + lg * 8);
                        co = Mf::k32(fm, fu, co);
                    }
                }
                bf16_t* bo = go + ((size_t)(t0 + (long)ch * CH) * H + h) * DV;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = a * 16 + lg * 4 + e;
                    if (full || ch * CH + r < len) bo[(unsigned)(r * H * DV + col)] = (bf16_t)(p.scale * co[e]);
                }
            }
            // S <- Pn*S0 + (Pn/Pm) (Kc^T U)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const auto fk = Mf::ld32(sKcT + (ct * 16 + ln) * LDC + s * 32 + lg * 8);
                    const auto fu = Mf::ld32(cU + ln * LDC + s * 32 + lg * 8);
                    acc = Mf::k32(fk, fu, acc);
                }
                const float4 pn = ld4(vec + DK + ct * 16 + lg * 4);
                const float4 pnm = ld4(vec + 2 * DK + ct * 16 + lg * 4);
                const f32x4 sv = rf_f4(4 * ct);
                f32x4 sn = {pn.x * sv[0] + pnm.x * acc[0], pn.y * sv[1] + pnm.y * acc[1],
                            pn.z * sv[2] + pnm.z * acc[2], pn.w * sv[3] + pnm.w * acc[3]};
                rf_set4(4 * ct, sn);
            }
        } else if (ch + 1 < nch) {
            p_gram(ch + 1);
        }
        __syncthreads();
    }

    if (pf_sink == 0x5a5a1234u && tid == 0x7fffffff) p.sT[0] = 0.f;  // keeps the prefetches
    if (consumer && p.sT) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.sT[sbase + (size_t)(ct * 16 + lg * 4 + e) * DV + col] = rf_f(4 * ct + e);
    }
}

template <int DK, int DVT>
static hipError_t launch_t(const KParams& p, hipStream_t stream) {
    using Lay = Lay3<DK, DVT>;
    static const hipError_t attr = hipFuncSetAttribute(
        (const void*)chunk_fwd_bf16_kernel<DK, DVT>, hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    const long grid = 8L * p.njt_all * ((p.units + 7) / 8);
    hipLaunchKernelGGL((chunk_fwd_bf16_kernel<DK, DVT>), dim3((unsigned)grid), dim3(Lay::NTH),
                       Lay::bytes, stream, p);
    return hipGetLastError();
}

// value-column tile widths this kernel supports
bool chunk_bf16_supports(int dvt) { return dvt == 16 || dvt == 32; }

hipError_t launch_chunk_bf16(const KParams& p, int dk, int dvt, hipStream_t stream) {
    if (dk == 128) return dvt == 16 ? launch_t<128, 16>(p, stream) : launch_t<128, 32>(p, stream);
    return dvt == 16 ? launch_t<64, 16>(p, stream) : launch_t<64, 32>(p, stream);
}

}  // namespace kda
