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
// Roles.  A workgroup owns one (unit, 16*NJT value columns).  Waves 0..3 are
// producers: they build chunk c+1's operands (decays, Kr, Qr, Kc, Kc^T), its
// Gram blocks (L, M) and the diagonal inverses D_a while the consumers work on
// chunk c.  Waves 4..4+NJT-1 are consumers: each keeps one 16-column slice of
// the fp32 state in registers and runs the state chain of chunk c (X, the
// solve, O, the next state).  Waves w and w+4 share a SIMD, so the consumers
// pair with producers 0 and 1 and producers 2 and 3 have a SIMD each; the
// D_a inverses go to producer 3.
// Everything a consumer reads from a producer is double-buffered by chunk
// parity except Kc^T and D, which are written in the consumer's own chunk.
// Two workgroup barriers per chunk:
//   segment 1: consumers  - Pm*S0, X and Qr (Pm*S0) of chunk c
//              producers  - write Kc^T(c); D_a(c); operands of chunk c+1
//   segment 2: consumers  - solve, O, next state (chunk c)
//              producers  - Gram blocks of chunk c+1
//
// Global memory is reached through buffer descriptors rebased per chunk whose
// range ends with the sequence's last row in the chunk: rows past the end of
// a sequence lie outside it, so their loads return zero and their stores are
// dropped.
#include "chunk_common.h"

namespace kda {

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    // raw buffer: stride 0, num_records = bytes, dword 3 = 32-bit data format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
template <int BYTES>
__device__ __forceinline__ void bload(uint32_t* dst, Rsrc r, uint32_t vo, uint32_t so) {
    if constexpr (BYTES == 8) {
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0);
        dst[0] = x[0]; dst[1] = x[1];
    } else {
        static_assert(BYTES % 16 == 0, "load width");
#pragma unroll
        for (int i = 0; i < BYTES / 16; ++i) {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, vo + 16 * i, so, 0);
            dst[4 * i] = x[0]; dst[4 * i + 1] = x[1]; dst[4 * i + 2] = x[2]; dst[4 * i + 3] = x[3];
        }
    }
}

template <int DK, int DVT>
struct Lay4 {
    static constexpr int NJT = DVT / 16;       // consumer waves
    static constexpr int NW = 4 + NJT;         // 4 producer waves first
    static constexpr int NTH = 64 * NW;
    static constexpr int CPL = DK / 16;        // key channels per producer lane
    static constexpr int LDK = DK + 8;         // bf16 pitch of [token][channel] tiles
    static constexpr int LDC = CH + 8;         // bf16 pitch of [*][token] tiles
    static constexpr int LDB = 16 + 8;         // bf16 pitch of packed 16x16 blocks
    static constexpr int LDL = 20;             // fp32 pitch of the diagonal blocks of L
    static constexpr int LDV = CH + 4;         // bf16 pitch of the V^T tile
    static constexpr int BLK = 16 * LDB;       // elements per packed block

    static constexpr size_t szTok = (size_t)CH * LDK * 2;
    // one parity buffer
    static constexpr size_t bKr = 0;
    static constexpr size_t bQr = bKr + szTok;
    static constexpr size_t bLo = bQr + szTok;                  // -L_ab, b < a: 6 blocks
    static constexpr size_t bM = bLo + (size_t)6 * BLK * 2;     // M_ab, b <= a: 10 blocks
    static constexpr size_t bVec = bM + (size_t)10 * BLK * 2;   // fp32 Pm, Pn, Pn/Pm [3][DK]
    static constexpr size_t bBeta = bVec + (size_t)3 * DK * 4;  // fp32 [64]
    static constexpr size_t bD = bBeta + CH * 4;                // D_a, 4 blocks row-major
    static constexpr size_t szBuf = (bD + (size_t)4 * BLK * 2 + 15) / 16 * 16;
    // single copies
    static constexpr size_t oKcT = 2 * szBuf;                   // [DK][LDC]
    static constexpr size_t oKc = oKcT + (size_t)DK * LDC * 2;  // [64][LDK], producers only
    static constexpr size_t oLd = oKc + szTok;                  // fp32 [4][16 cols][LDL], producer 3
    static constexpr size_t oVT = oLd + (size_t)4 * 16 * LDL * 4;  // bf16 V^T [DVT][LDV]
    // consumer-private scratch
    static constexpr size_t cSP = 0;                            // [16][LDK] bf16: (Pm*S0)^T
    static constexpr size_t cU = cSP + (size_t)16 * LDK * 2;    // [16][LDC] bf16: U^T
    static constexpr size_t szC = (cU + (size_t)16 * LDC * 2 + 15) / 16 * 16;
    static constexpr size_t oCons = oVT + (size_t)DVT * LDV * 2;
    static constexpr size_t bytes = oCons + NJT * szC;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    bf16x2v h;
    h[0] = (bf16_t)a; h[1] = (bf16_t)b;
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// Element offset of (row, channel) in a [64][LDK] token tile.  The 16-byte
// column chunks of a row are XOR-swizzled by (row / 16) mod 4: a producer
// lane writes rows 4 apart (16-byte stores), and unswizzled those rows would
// share four bank groups; swizzled, the 16 lanes of a store and the 16 rows of
// a matrix-core fragment read each hit distinct banks.
template <int LDK>
__device__ __forceinline__ int tok_off(int row, int ch) {
    return row * LDK + ((((ch >> 3) ^ (row >> 4)) & 3) | ((ch >> 3) & ~3)) * 8 + (ch & 7);
}
// the same value in every lane of this lane's 16-lane row: lane LANE's
template <int LANE>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + LANE, 0xf, 0xf, false));
}

// A copy of x that the compiler cannot see through.  Values derived from it
// are recomputed where they are used instead of being hoisted out of the chunk
// loop and kept live (or spilled) for the whole kernel.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}
// value of lane l - d inside this lane's 16-lane row, or `old` for the first d lanes
template <int D>
__device__ __forceinline__ float row_shr(float x, float old) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x),
                                                      0x110 + D, 0xf, 0xf, false));
}
// x * (x of lane l - D) inside this lane's 16-lane row; the first D lanes of the
// row keep x (their DPP source is outside the row and, with bound_ctrl clear,
// the lane is not written).  One DPP multiply; the s_nop covers the wait
// states a DPP read needs after a VALU write of its source.
#define KDA_MUL_ROW_SHR(NAME, D)                                                              \
    __device__ __forceinline__ float NAME(float x) {                                          \
        float r = x;                                                                          \
        asm volatile("s_nop 1\n\tv_mul_f32_dpp %0, %1, %0 row_shr:" #D                        \
                     " row_mask:0xf bank_mask:0xf" : "+v"(r) : "v"(x));                       \
        return r;                                                                             \
    }
KDA_MUL_ROW_SHR(mul_row_shr1, 1)
KDA_MUL_ROW_SHR(mul_row_shr2, 2)
KDA_MUL_ROW_SHR(mul_row_shr4, 4)
KDA_MUL_ROW_SHR(mul_row_shr8, 8)
#undef KDA_MUL_ROW_SHR

template <int DK, int DVT>
__global__ __launch_bounds__((Lay4<DK, DVT>::NTH), 1) void chunk_fwd_bf16_kernel(KParams p) {
    using L = Lay4<DK, DVT>;
    using Mf = Mma<bf16_t>;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDB = L::LDB, LDL = L::LDL, BLK = L::BLK;
    constexpr int CPL = L::CPL;
    constexpr int NCT = DK / 16;          // 16-row tiles of a state slice

    // Values a wave carries from one chunk to the next live in one register
    // array shared by the two roles (a wave keeps its role for the whole
    // kernel), so the allocation is the larger of the two sets, not the sum.
    //   producer: raw q rows | raw k rows | raw alpha rows | Kc^T bf16 pairs | beta | raw v
    //   consumer: state | beta-scaled X | Qr(Pm S0)
    constexpr int QO = 0, KO = 2 * CPL, AO = 4 * CPL, TO = 8 * CPL, BO = 10 * CPL, VPO = BO + 1;
    constexpr int YO = DK / 4, IO = DK / 4 + 16;
    constexpr int RFN = (VPO + 4 > IO + 16) ? VPO + 4 : IO + 16;
    constexpr int CPV = DVT / 16;  // value columns per producer lane in the V^T tile
    static_assert(4 * NCT == YO, "register file layout");

    extern __shared__ __align__(16) unsigned char smem[];
    auto buf = [&](int par, size_t off) { return smem + par * L::szBuf + off; };
    bf16_t* sKcT = reinterpret_cast<bf16_t*>(smem + L::oKcT);
    bf16_t* sKc = reinterpret_cast<bf16_t*>(smem + L::oKc);
    float* sLd = reinterpret_cast<float*>(smem + L::oLd);
    bf16_t* sVT = reinterpret_cast<bf16_t*>(smem + L::oVT);

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
    const bool producer = w < 4;

    // byte strides of one token row
    const uint32_t rsq = (uint32_t)H * DK * 2, rsa = (uint32_t)H * DK * 4;
    const uint32_t rsb = (uint32_t)H * 4, rsv = (uint32_t)H * DV * 2;

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
    // Lane (cq = l/16, rg = l%16) of producer pw owns key channels
    // pc0..pc0+CPL-1 and rows 4rg..4rg+3; a 16-lane row holds one channel
    // group, so the scan over row groups runs inside DPP rows.
    const int pw = w;
    const int rg = ln, cq = lg;
    const int pc0 = pw * (DK / 4) + cq * CPL;
    const int pr0 = rg * 4;
    const bf16_t* __restrict__ gq = static_cast<const bf16_t*>(p.q);
    const bf16_t* __restrict__ gk = static_cast<const bf16_t*>(p.k);
    const float* __restrict__ ga = p.alpha;
    const float* __restrict__ gb = p.beta;
    const uint32_t qoff = (uint32_t)pr0 * rsq + (uint32_t)pc0 * 2;
    const uint32_t aoff = (uint32_t)pr0 * rsa + (uint32_t)pc0 * 4;
    // V^T tile: lane (vq = 4 pw + l/16, vc = l%16) moves rows 4vq..4vq+3 of columns vc0..vc0+CPV-1
    const bf16_t* __restrict__ gv = static_cast<const bf16_t*>(p.v);
    const int vq = pw * 4 + lg, vc0 = ln * CPV;
    const uint32_t vpoff = (uint32_t)(4 * vq) * rsv + (uint32_t)vc0 * 2;

    auto p_load = [&](int ch) {  // raw q, k, alpha, beta rows of chunk ch; rows past the end read as zero
        const size_t e0 = ((size_t)(t0 + (long)ch * CH) * H + h) * DK;
        // rows of this chunk inside the sequence (0 past the last chunk: every
        // load then falls outside the range, reads nothing and returns zero;
        // issuing the loads anyway keeps the count of loads in flight the same
        // on every path, so the waits for them stay exact)
        const int nr = __builtin_amdgcn_readfirstlane(max(0, min(len - ch * CH, CH)));
        const Rsrc rq = make_rsrc(gq + e0, (uint32_t)nr * rsq);
        const Rsrc rk = make_rsrc(gk + e0, (uint32_t)nr * rsq);
        const Rsrc ra = make_rsrc(ga + e0, (uint32_t)nr * rsa);
        const uint32_t qo = opaque(qoff), ao = opaque(aoff);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            bload<CPL * 2>(&RF[QO + rr * (CPL / 2)], rq, qo + rr * rsq, 0);
            bload<CPL * 2>(&RF[KO + rr * (CPL / 2)], rk, qo + rr * rsq, 0);
            bload<CPL * 4>(&RF[AO + rr * CPL], ra, ao + rr * rsa, 0);
        }
        const Rsrc rb = make_rsrc(gb + ((size_t)(t0 + (long)ch * CH) * H + h), (uint32_t)nr * rsb);
        RF[BO] = __builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)l * rsb, 0, 0);
    };
    // the consumers' V slice of chunk ch: rows 4vq..4vq+3, columns vc0..vc0+CPV-1
    auto p_load_v = [&](int ch) {
        const int nr = __builtin_amdgcn_readfirstlane(max(0, min(len - ch * CH, CH)));
        const Rsrc rv = make_rsrc(gv + ((size_t)(t0 + (long)ch * CH) * H + h) * DV + jt * DVT,
                                  (uint32_t)nr * rsv);
        const uint32_t vo = opaque(vpoff);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            if constexpr (CPV == 2)
                RF[VPO + rr] = __builtin_amdgcn_raw_buffer_load_b32(rv, vo + rr * rsv, 0, 0);
            else
                RF[VPO + rr] = __builtin_amdgcn_raw_buffer_load_b16(rv, vo + rr * rsv, 0, 0);
        }
    };

    // decayed operands of chunk ch into parity buffer ch & 1 (Kc^T kept in RF)
    auto p_operands = [&](int ch) {
        // lane coordinates recomputed here (see opaque()) rather than kept live
        const int lx = (int)opaque((uint32_t)l);
        const int rg = lx & 15, cq = lx >> 4;
        const int pc0 = pw * (DK / 4) + cq * CPL, pr0 = rg * 4;
        const int par = ch & 1;
        const int nval = len - ch * CH;
        if (nval < CH) {  // alpha of rows past the end of the sequence is 1
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                if (pr0 + rr >= nval)
#pragma unroll
                    for (int c = 0; c < CPL; ++c) RF[AO + rr * CPL + c] = __float_as_uint(1.f);
        }
        float pr[4][CPL];  // running product over the lane's rows
        float inc[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float run = rf_f(AO + c);
            pr[0][c] = run;
#pragma unroll
            for (int rr = 1; rr < 4; ++rr) { run *= rf_f(AO + rr * CPL + c); pr[rr][c] = run; }
            inc[c] = run;
        }
        // inclusive product over row groups 0..rg of the same channels
#pragma unroll
        for (int c = 0; c < CPL; ++c) inc[c] = mul_row_shr1(inc[c]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) inc[c] = mul_row_shr2(inc[c]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) inc[c] = mul_row_shr4(inc[c]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) inc[c] = mul_row_shr8(inc[c]);
        // Pm, 1/Pm and Pn from row groups 7 and 15 of the same channel group
        float ri[CPL], pm[CPL], ipm[CPL], pn[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            ri[c] = fast_rcp(inc[c]);  // 1 / P through row pr0 + 3
            pm[c] = row_bcast<7>(inc[c]);
            ipm[c] = row_bcast<7>(ri[c]);
            pn[c] = row_bcast<15>(inc[c]);
        }
        float f[CPL], g[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            f[c] = row_shr<1>(inc[c], 1.f) * ipm[c];  // P through row pr0 - 1, over Pm
            g[c] = pm[c] * ri[c];                       // Pm / P through row pr0 + 3
        }
        if (rg == 0) {
            float* vec = reinterpret_cast<float*>(buf(par, L::bVec));
#pragma unroll
            for (int c = 0; c < CPL; c += 4) {
                *reinterpret_cast<float4*>(vec + pc0 + c) = make_float4(pm[c], pm[c + 1], pm[c + 2], pm[c + 3]);
                *reinterpret_cast<float4*>(vec + DK + pc0 + c) = make_float4(pn[c], pn[c + 1], pn[c + 2], pn[c + 3]);
                *reinterpret_cast<float4*>(vec + 2 * DK + pc0 + c) =
                    make_float4(pn[c] * ipm[c], pn[c + 1] * ipm[c + 1], pn[c + 2] * ipm[c + 2], pn[c + 3] * ipm[c + 3]);
            }
        }
        if (pw == 0) reinterpret_cast<float*>(buf(par, L::bBeta))[l] = rf_f(BO);
        bf16_t* kr_b = reinterpret_cast<bf16_t*>(buf(par, L::bKr));
        bf16_t* qr_b = reinterpret_cast<bf16_t*>(buf(par, L::bQr));
        // rows from the last to the first: g_r = Pm / P_r = g_{r+1} * alpha_{r+1}
        uint32_t kcp[CPL / 2];  // Kc of row rr + 1 (the odd row of the current pair)
#pragma unroll
        for (int rr = 3; rr >= 0; --rr) {
            uint32_t kr[CPL / 2], qr[CPL / 2], kc[CPL / 2];
#pragma unroll
            for (int i = 0; i < CPL / 2; ++i) {
                const uint32_t kw = RF[KO + rr * (CPL / 2) + i], qw = RF[QO + rr * (CPL / 2) + i];
                const int c0 = 2 * i, c1 = 2 * i + 1;
                if (rr < 3) {
                    g[c0] *= rf_f(AO + (rr + 1) * CPL + c0);
                    g[c1] *= rf_f(AO + (rr + 1) * CPL + c1);
                }
                const float r0 = pr[rr][c0] * f[c0], r1 = pr[rr][c1] * f[c1];
                const float k0 = lo_f(kw), k1 = hi_f(kw);
                kr[i] = pack2(k0 * r0, k1 * r1);
                qr[i] = pack2(lo_f(qw) * r0, hi_f(qw) * r1);
                kc[i] = pack2(k0 * g[c0], k1 * g[c1]);
                if (rr & 1) {
                    kcp[i] = kc[i];
                } else {  // Kc^T pairs of channels c0, c1: rows (rr, rr + 1)
                    RF[TO + 2 * c0 + (rr >> 1)] = __builtin_amdgcn_perm(kcp[i], kc[i], 0x05040100u);
                    RF[TO + 2 * c1 + (rr >> 1)] = __builtin_amdgcn_perm(kcp[i], kc[i], 0x07060302u);
                }
            }
            const int to = tok_off<LDK>(pr0 + rr, pc0);
            if constexpr (CPL == 8) {
                *reinterpret_cast<uint4*>(kr_b + to) = make_uint4(kr[0], kr[1], kr[2], kr[3]);
                *reinterpret_cast<uint4*>(qr_b + to) = make_uint4(qr[0], qr[1], qr[2], qr[3]);
                *reinterpret_cast<uint4*>(sKc + to) = make_uint4(kc[0], kc[1], kc[2], kc[3]);
            } else {
                *reinterpret_cast<uint2*>(kr_b + to) = make_uint2(kr[0], kr[1]);
                *reinterpret_cast<uint2*>(qr_b + to) = make_uint2(qr[0], qr[1]);
                *reinterpret_cast<uint2*>(sKc + to) = make_uint2(kc[0], kc[1]);
            }
        }
    };

    // V^T of the chunk whose V rows are in RF: rows 4vq..4vq+3 of column vc0 (+1) as 8-byte runs
    auto p_write_vt = [&]() {
        const int lx = (int)opaque((uint32_t)l);
        const int vq = pw * 4 + (lx >> 4), vc0 = (lx & 15) * CPV;
        const uint32_t lo01 = __builtin_amdgcn_perm(RF[VPO + 1], RF[VPO], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(RF[VPO + 3], RF[VPO + 2], 0x05040100u);
        *reinterpret_cast<uint2*>(sVT + vc0 * L::LDV + 4 * vq) = make_uint2(lo01, lo23);
        if constexpr (CPV == 2) {
            const uint32_t hi01 = __builtin_amdgcn_perm(RF[VPO + 1], RF[VPO], 0x07060302u);
            const uint32_t hi23 = __builtin_amdgcn_perm(RF[VPO + 3], RF[VPO + 2], 0x07060302u);
            *reinterpret_cast<uint2*>(sVT + (vc0 + 1) * L::LDV + 4 * vq) = make_uint2(hi01, hi23);
        }
    };

    auto p_write_kct = [&]() {
        // lane coordinates recomputed here (see opaque()) rather than kept live
        const int lx = (int)opaque((uint32_t)l);
        const int rg = lx & 15, cq = lx >> 4;
        const int pc0 = pw * (DK / 4) + cq * CPL, pr0 = rg * 4;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            *reinterpret_cast<uint2*>(sKcT + (pc0 + c) * LDC + pr0) = make_uint2(RF[TO + 2 * c], RF[TO + 2 * c + 1]);
    };

    // Gram blocks of chunk ch, then D_a = (I + L_aa)^{-1}.  Producer 3 takes the
    // four diagonal blocks (a, a) and inverts them; producers 0..2 take two of
    // the six blocks below the diagonal each.
    auto p_gram = [&](int ch) {
        const int lx = (int)opaque((uint32_t)l);
        const int ln = lx & 15, lg = lx >> 4;
        const int par = ch & 1;
        const bf16_t* kr_b = reinterpret_cast<const bf16_t*>(buf(par, L::bKr));
        const bf16_t* qr_b = reinterpret_cast<const bf16_t*>(buf(par, L::bQr));
        bf16_t* lo_b = reinterpret_cast<bf16_t*>(buf(par, L::bLo));
        bf16_t* m_b = reinterpret_cast<bf16_t*>(buf(par, L::bM));
        const float* beta = reinterpret_cast<const float*>(buf(par, L::bBeta));
        // lane holds A[r = 16a + ln][i = 16b + 4lg + e] (and M likewise)
        auto gram_block = [&](int a, int b, f32x4& cA, f32x4& cM) {
            cA = zero4(); cM = zero4();
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                const auto fa = Mf::ld32(sKc + tok_off<LDK>(b * 16 + ln, s * 32 + lg * 8));
                const auto fk = Mf::ld32(kr_b + tok_off<LDK>(a * 16 + ln, s * 32 + lg * 8));
                const auto fq = Mf::ld32(qr_b + tok_off<LDK>(a * 16 + ln, s * 32 + lg * 8));
                cA = Mf::k32(fa, fk, cA);
                cM = Mf::k32(fa, fq, cM);
            }
        };
        if (pw == 3) {
            f32x4 cA[4], cM[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) gram_block(a, a, cA[a], cM[a]);
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const float br = beta[a * 16 + ln];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = lg * 4 + e;  // L_aa stored column-major, fp32
                    sLd[(a * 16 + i) * LDL + ln] = (i < ln) ? br * cA[a][e] : 0.f;
                }
                f32x4 mm;
#pragma unroll
                for (int e = 0; e < 4; ++e) mm[e] = (lg * 4 + e <= ln) ? cM[a][e] : 0.f;
                Mf::st4(m_b + (a * (a + 3) / 2) * BLK + ln * LDB + lg * 4, mm);
            }
        } else {
            // blocks (a, b), b < a: job j = a (a - 1) / 2 + b of the six, two per producer
            f32x4 cA[2], cM[2];
            int aa[2], bb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int j = pw + 3 * t;  // (1,0) (2,0) (2,1) | (3,0) (3,1) (3,2)
                aa[t] = j >= 3 ? 3 : j >= 1 ? 2 : 1;
                bb[t] = j - aa[t] * (aa[t] - 1) / 2;
                gram_block(aa[t], bb[t], cA[t], cM[t]);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int a = aa[t], b = bb[t];
                const float br = beta[a * 16 + ln];
                f32x4 lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) lo[e] = -br * cA[t][e];
                Mf::st4(lo_b + (a * (a - 1) / 2 + b) * BLK + ln * LDB + lg * 4, lo);
                Mf::st4(m_b + (a * (a + 1) / 2 + b) * BLK + ln * LDB + lg * 4, cM[t]);
            }
        }
    };

    // D_a = (I + L_aa)^{-1} of chunk ch: lane (block lg, column ln), right-looking, fp32
    auto p_dsolve = [&](int ch) {
        bf16_t* sD = reinterpret_cast<bf16_t*>(buf(ch & 1, L::bD));
        const uint32_t lnx = opaque(ln);
        float xs[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) xs[r] = (r == (int)lnx) ? 1.f : 0.f;
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
        for (int r = 0; r < 16; ++r) sD[lg * BLK + r * LDB + ln] = (bf16_t)xs[r];
    };

    // ------------------------------------------------------------ consumers
    const int cj = w - 4;                    // consumer column tile
    const int colw = jt * DVT + cj * 16;     // first value column of this wave
    const int col = colw + ln;               // this lane's value column
    unsigned char* cbase = smem + L::oCons + (producer ? 0 : cj) * L::szC;
    bf16_t* cSP = reinterpret_cast<bf16_t*>(cbase + L::cSP);
    bf16_t* cU = reinterpret_cast<bf16_t*>(cbase + L::cU);
    bf16_t* __restrict__ go = static_cast<bf16_t*>(p.o);
    const size_t sbase = ((size_t)wi.seq * H + h) * DK * DV;
    const uint32_t voff = (uint32_t)ln * 2 + (uint32_t)lg * 4 * rsv;  // row 4lg, column col

    // The two roles run separate loops with the same barriers (two per chunk
    // plus two in the prologue; nch is uniform over the workgroup), so each
    // role's registers are allocated on their own.
    //   producers, segment 1: Kc^T(c); operands of c+1; q, k, alpha, beta loads of c+2
    //   producers, segment 2: Gram blocks and D of c+1; V^T(c+1); V loads of c+2
    // Every producer step runs unconditionally.  Past the last chunk its loads
    // fall outside their descriptors and return zero, and it writes zero
    // operands into the parity buffer nobody reads any more; in exchange no
    // path skips a load or a use of loaded registers, which keeps the waits
    // for the loads in flight exact instead of draining the queue.
    if (producer) {
        p_load(0);
        p_load_v(0);
        p_operands(0);
        p_load(1);
        __syncthreads();
        p_gram(0);
        if (pw == 3) { wave_sync_lds(); p_dsolve(0); }
        p_write_vt();
        p_load_v(1);
        __syncthreads();
        for (int ch = 0; ch < nch; ++ch) {
            // segment 1
            p_write_kct();  // Kc^T of chunk ch (its Kc came with the operands one chunk ago)
            p_operands(ch + 1);
            p_load(ch + 2);
            __syncthreads();
            // segment 2
            p_gram(ch + 1);
            if (pw == 3) { wave_sync_lds(); p_dsolve(ch + 1); }
            p_write_vt();
            p_load_v(ch + 2);
            __syncthreads();
        }
        return;
    }

    // The consumers carry the serial state chain: let the SIMD arbiter prefer
    // them over the producer waves they share a SIMD with.
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        if (p.s0) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                RF[4 * ct + e] = __float_as_uint(p.s0[sbase + (size_t)(ct * 16 + lg * 4 + e) * DV + col]);
        }
    }
    __syncthreads();
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int par = ch & 1;
        // ======================= segment 1 =======================
        {
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
        const bf16_t* vt = sVT;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4 cx = zero4(), co = zero4();
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                const auto fs = Mf::ld32(cSP + ln * LDK + s * 32 + lg * 8);
                const auto fk = Mf::ld32(kr_b + tok_off<LDK>(a * 16 + ln, s * 32 + lg * 8));
                const auto fq = Mf::ld32(qr_b + tok_off<LDK>(a * 16 + ln, s * 32 + lg * 8));
                cx = Mf::k32(fk, fs, cx);
                co = Mf::k32(fq, fs, co);
            }
            const float4 b4 = ld4(beta + a * 16 + lg * 4);
            const uint2 v4 = *reinterpret_cast<const uint2*>(vt + (cj * 16 + ln) * L::LDV + a * 16 + lg * 4);
            // beta_r (v_r - (Kr Pm S0)_r); rows past the end have v = beta = 0
            f32x4 y;
            y[0] = b4.x * (lo_f(v4.x) - cx[0]);
            y[1] = b4.y * (hi_f(v4.x) - cx[1]);
            y[2] = b4.z * (lo_f(v4.y) - cx[2]);
            y[3] = b4.w * (hi_f(v4.y) - cx[3]);
            rf_set4(YO + 4 * a, y);
            rf_set4(IO + 4 * a, co);
        }
        }
        __syncthreads();
        // ======================= segment 2 =======================
        {
        const bf16_t* lo_b = reinterpret_cast<const bf16_t*>(buf(par, L::bLo));
        const bf16_t* m_b = reinterpret_cast<const bf16_t*>(buf(par, L::bM));
        const float* vec = reinterpret_cast<const float*>(buf(par, L::bVec));
        // U_a = D_a (Y_a - sum_{b<a} L_ab U_b); lo_b holds -L_ab
        f32x4 U[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4 acc = rf_f4(YO + 4 * a);
#pragma unroll
            for (int b = 0; b < a; ++b) {
                const auto fl = Mf::ld16(lo_b + (a * (a - 1) / 2 + b) * BLK + ln * LDB + lg * 4);
                acc = Mf::k16(fl, Mf::pack16(U[b]), acc);
            }
            const auto fd = Mf::ld16(reinterpret_cast<const bf16_t*>(buf(par, L::bD)) + a * BLK + ln * LDB + lg * 4);
            U[a] = Mf::k16(fd, Mf::pack16(acc), zero4());
            Mf::st4(cU + ln * LDC + a * 16 + lg * 4, U[a]);
        }
        wave_sync_lds();
        // O_a = scale (OI_a + sum_{b<=a} M_ab U_b), k-steps of 32 tokens
        const Rsrc ro = make_rsrc(go + ((size_t)(t0 + (long)ch * CH) * H + h) * DV + colw,
                                  (uint32_t)min(len - ch * CH, CH) * rsv);
        const uint32_t ob = opaque(voff);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4 co = rf_f4(IO + 4 * a);
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
#pragma unroll
            for (int e = 0; e < 4; ++e)
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (bf16_t)(p.scale * co[e])),
                                                      ro, ob + (uint32_t)(a * 16 + e) * rsv, 0, 0);
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
        }
        __syncthreads();
    }

    if (p.sT) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.sT[sbase + (size_t)(ct * 16 + lg * 4 + e) * DV + col] = rf_f(4 * ct + e);
    }
}

template <int DK, int DVT>
static hipError_t launch_t(const KParams& p, hipStream_t stream) {
    using Lay = Lay4<DK, DVT>;
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
