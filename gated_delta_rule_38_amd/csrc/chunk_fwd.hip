// chunk_fwd.hip -- chunk-wise KDA forward on gfx950 matrix cores.
//
// Method: the chunk-wise mode of bugfactory.tech news 3610, fifth paragraph
// (intra-chunk transitions as matrix products with precomputed "A" matrices)
// and the chunk-parallel scheme on the kongchang.com page, section
// "硬件效率的优化策略" (parallel products inside a chunk, the state carried
// from chunk to chunk), applied to the update equation of "Kimi Delta
// Attention", section "KDA 的更新式".  The chunk identities are derived from
// that equation (the pages do not print them):
//
// For a chunk of C = 64 tokens with start state S0 and P_r the running product
// of alpha over tokens 0..r of the chunk (per key channel), the state after
// token r is S_r = Diag(P_r) S0 + sum_{i<=r} Diag(P_r/P_i) k_i u_i^T with the
// written pseudo-values u_r = beta_r (v_r - S~_r^T k_r).  Collecting rows:
//     (I + Diag(beta) A) U = Diag(beta) (V - Kg S0),  A_ri = sum_c k_rc k_ic P_rc/P_ic (i<r)
// so U = T (V - Kg S0) with T = (I + Diag(beta) A)^{-1} Diag(beta), and
//     O  = scale ((Q*P) S0 + M U),   M_ri = sum_c q_rc k_ic P_rc/P_ic (i<=r)
//     S_C = Diag(P_63) S0 + (K * P_63/P)^T U.
// Decay factors are referenced to the middle of the chunk (Pm = P_31) so that
// the two Gram factors K*P/Pm and K*Pm/P only span alpha's product over a half
// chunk (a chunk whose half-chunk product falls below 2^-100 in some channel
// sends its work item to the exact token walk of chunk_walk.h):
//     Kr = K*P/Pm, Qr = Q*P/Pm, Kc = K*Pm/P,  A = tril_-1(Kr Kc^T), M = tril(Qr Kc^T)
//     X = V - Kr (Pm*S0),  OI = Qr (Pm*S0),  U = T X
//     O = scale (OI + M U),  S_C = Pn*S0 + (Pn/Pm) * (Kc^T U)
// where "Pm*S0" scales row c of S0 by Pm_c.  Past the end of a sequence the
// chunk is padded with q = k = v = 0, beta = 0, alpha = 1, an exact no-op.
//
// T is formed blockwise over 16-token blocks: the four diagonal blocks are
// inverted by forward substitution in fp32 on the vector ALUs, and each
// off-diagonal block follows from T_ab = -D_a sum_{j=b}^{a-1} L_aj T_jb, one
// column block per wavefront, on the matrix cores.
//
// Work decomposition.  The value columns of S evolve independently (the
// transition acts on the key side), so a workgroup owns one (unit, value-
// column tile of DVT columns) and walks that unit's chunks in order with its
// state slice in registers.  Everything that does not depend on the value
// columns (decays, Gram matrices, T) is recomputed by every column tile of a
// unit; tiles of one unit are placed on the same XCD so their shared q, k,
// alpha reads hit the same L2.
#include "chunk_walk.h"

#include <mutex>

namespace kda {

constexpr int NTH = 256;

template <typename Top, int DK, int DVT>
struct ChunkLayout {
    static constexpr int ES = sizeof(Top);
    // fp32 operands at dk = 128 do not fit twice in LDS: the Gram's Kc
    // fragments are then gathered from the channel-major copy instead.
    static constexpr bool KCT_ONLY = (ES == 4 && DK == 128);
    static constexpr int PAD = 16 / ES;      // one 16-byte pad per row
    static constexpr int LDK = DK + PAD;     // pitch of [token][channel] tiles
    static constexpr int LDC = CH + PAD;     // pitch of [*][token] tiles
    static constexpr int LDD = 16 + PAD;     // pitch of 16x16 blocks
    static constexpr int LDL = 20;           // pitch of the fp32 diagonal blocks of L
    static constexpr int NJT = DVT / 16;     // 16-column tiles of the slice
    static constexpr int NCT = DK / 16;      // 16-row tiles of the state
    static constexpr int NST = NCT * NJT;    // state tiles
    static constexpr int STW = (NST + 3) / 4;  // state tiles per wavefront

    // region A, phases 0-1: chunk operands
    static constexpr size_t oKr = 0;
    static constexpr size_t oQr = oKr + (size_t)CH * LDK * ES;
    static constexpr size_t oKc = oQr + (size_t)CH * LDK * ES;
    static constexpr size_t oSP = oKc + (KCT_ONLY ? 0 : (size_t)CH * LDK * ES);
    static constexpr size_t endA1 = oSP + (size_t)DVT * LDK * ES;
    // region A, phases 2-4 (overlays the above)
    static constexpr size_t oTm = 0;
    static constexpr size_t oU = oTm + (size_t)CH * LDC * ES;
    static constexpr size_t oDr = oU + (size_t)DVT * LDC * ES;     // [4 waves][4][16][LDD]
    static constexpr size_t oDc = oDr + (size_t)4 * 4 * 16 * LDD * ES;
    static constexpr size_t endA2 = oDc + (size_t)4 * 4 * 16 * LDD * ES;
    static constexpr size_t endA = endA1 > endA2 ? endA1 : endA2;
    // region B
    static constexpr size_t oKcT = (endA + 255) / 256 * 256;
    static constexpr size_t oMm = oKcT + (size_t)DK * LDC * ES;
    static constexpr size_t oX = oMm + (size_t)CH * LDC * ES;
    static constexpr size_t oLo = oX + (size_t)DVT * LDC * ES;
    static constexpr size_t oLd = oLo + (size_t)CH * LDC * ES;        // fp32 [4][16][LDL]
    static constexpr size_t oTot = oLd + (size_t)4 * 16 * LDL * 4;    // fp32 [4][DK]
    static constexpr size_t oBeta = oTot + (size_t)4 * DK * 4;        // fp32 [64]
    static constexpr size_t oBad = oBeta + CH * 4;                    // u32 [4] out-of-range flags
    static constexpr size_t bytes = oBad + 16;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// CPT = DK/64 consecutive channels of one token row, kept in registers in
// their stored form between the prefetch and the use one chunk later, so the
// loads stay in flight across the intervening work.
template <typename Tin, int CPT>
struct RawRow;
template <> struct RawRow<bf16_t, 1> {
    typedef uint16_t T;
    static __device__ __forceinline__ T ld(const bf16_t* p) {
        return *reinterpret_cast<const uint16_t*>(p);
    }
    static __device__ __forceinline__ void unpack(T w, float* x) {
        x[0] = __uint_as_float(uint32_t(w) << 16);
    }
};
template <> struct RawRow<bf16_t, 2> {
    typedef uint32_t T;
    static __device__ __forceinline__ T ld(const bf16_t* p) {
        return *reinterpret_cast<const uint32_t*>(p);
    }
    static __device__ __forceinline__ void unpack(T w, float* x) {
        x[0] = __uint_as_float(w << 16);
        x[1] = __uint_as_float(w & 0xffff0000u);
    }
};
template <> struct RawRow<float, 1> {
    typedef float T;
    static __device__ __forceinline__ T ld(const float* p) { return *p; }
    static __device__ __forceinline__ T splat(float a) { return a; }
    static __device__ __forceinline__ T pack(const float* x) { return x[0]; }
    static __device__ __forceinline__ void unpack(T w, float* x) { x[0] = w; }
};
template <> struct RawRow<float, 2> {
    typedef float2 T;
    static __device__ __forceinline__ T ld(const float* p) {
        return *reinterpret_cast<const float2*>(p);
    }
    static __device__ __forceinline__ T splat(float a) { return make_float2(a, a); }
    static __device__ __forceinline__ T pack(const float* x) { return make_float2(x[0], x[1]); }
    static __device__ __forceinline__ void unpack(T w, float* x) { x[0] = w.x; x[1] = w.y; }
};


// A k32 fragment gathered with a stride (8 scalar LDS reads), used where the
// row-contiguous copy of an operand is not kept.
template <typename Top>
__device__ __forceinline__ typename Mma<Top>::F32 gather32(const Top* p, int stride);
template <>
__device__ __forceinline__ Mma<float>::F32 gather32<float>(const float* p, int stride) {
    return Mma<float>::F32{make_float4(p[0], p[stride], p[2 * stride], p[3 * stride]),
                           make_float4(p[4 * stride], p[5 * stride], p[6 * stride], p[7 * stride])};
}
template <>
__device__ __forceinline__ Mma<bf16_t>::F32 gather32<bf16_t>(const bf16_t* p, int stride) {
    Mma<bf16_t>::F32 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = p[e * stride];
    return f;
}


// ckpt (may be NULL): the state at the start of every chunk of every unit, and
// after its last chunk, for the chunk-wise backward.  Unit (seq, h) uses slots
// slot0 .. slot0 + nch with slot0 = t0 / 64 + 2 seq (t0 its first token), so
// sequences never share a slot; slot s of head h is the float32 [dk][dv] block
// at ((s * H + h) * dk * dv).  With p.o == NULL no output is formed.
template <typename Tin, int DK, int DVT>
__global__ __launch_bounds__(NTH, 1) void chunk_fwd_kernel(KParams p, float* __restrict__ ckpt) {
    using Top = Tin;
    using L = ChunkLayout<Top, DK, DVT>;
    using M = Mma<Top>;
    constexpr int CPT = DK / 64;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDD = L::LDD, NJT = L::NJT;
    constexpr int NST = L::NST, STW = L::STW, NJT_S = L::NJT;

    extern __shared__ __align__(16) unsigned char smem[];
    Top* sKr = reinterpret_cast<Top*>(smem + L::oKr);
    Top* sQr = reinterpret_cast<Top*>(smem + L::oQr);
    Top* sKc = reinterpret_cast<Top*>(smem + L::oKc);
    Top* sSP = reinterpret_cast<Top*>(smem + L::oSP);
    Top* sTm = reinterpret_cast<Top*>(smem + L::oTm);
    Top* sU = reinterpret_cast<Top*>(smem + L::oU);
    Top* sDr = reinterpret_cast<Top*>(smem + L::oDr);
    Top* sDc = reinterpret_cast<Top*>(smem + L::oDc);
    Top* sKcT = reinterpret_cast<Top*>(smem + L::oKcT);
    Top* sMm = reinterpret_cast<Top*>(smem + L::oMm);
    Top* sX = reinterpret_cast<Top*>(smem + L::oX);
    Top* sLo = reinterpret_cast<Top*>(smem + L::oLo);
    float* sLd = reinterpret_cast<float*>(smem + L::oLd);
    float* sTot = reinterpret_cast<float*>(smem + L::oTot);
    float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);
    uint32_t* sBad = reinterpret_cast<uint32_t*>(smem + L::oBad);
    static_assert(WalkShape<DVT, NTH, false>::lds_bytes <= L::oBad, "walk LDS");

    const WorkItem wi = decode_work(p);
    if (!wi.valid) return;
    const int H = p.H, h = wi.h, seq = wi.seq, jt = wi.jt, len = wi.len;
    const long t0 = wi.t0;
    const int DV = p.dv;
    const Tin* __restrict__ gq = static_cast<const Tin*>(p.q);
    const Tin* __restrict__ gk = static_cast<const Tin*>(p.k);
    const Tin* __restrict__ gv = static_cast<const Tin*>(p.v);
    const float* __restrict__ ga = static_cast<const float*>(p.alpha);
    const Tin* __restrict__ gg = static_cast<const Tin*>(p.alpha);  // gate logits
    const float* __restrict__ gb = p.beta;
    const int gate = p.gate;
    const bool gl = p.fuse & FUSE_GATE_LOGITS, qn = p.fuse & FUSE_QK_L2NORM;
    Tin* __restrict__ go = static_cast<Tin*>(p.o);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront (uniform)
    const int l = tid & 63;     // lane
    const int ln = l & 15;      // C-layout column / fragment row
    const int lg = l >> 4;      // lane group
    const int col0 = jt * DVT;  // first value column of this slice

    // ---- state slice in C-layout registers: wave w owns tiles w, w+4, ... ----
    f32x4 S[STW];
    const size_t sbase = ((size_t)seq * H + h) * DK * DV;
#pragma unroll
    for (int i = 0; i < STW; ++i) {
        const int st = w + 4 * i;
        S[i] = zero4();
        if (st < NST && p.s0) {
            const int ct = st / NJT_S, jj = st % NJT_S;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[i][e] = p.s0[sbase + (size_t)(ct * 16 + lg * 4 + e) * DV + col0 + jj * 16 + ln];
        }
    }

    // M's blocks above the diagonal are read by the 32-wide k-steps and must
    // be zero; nothing else writes them.
    for (int idx = tid; idx < CH * CH; idx += NTH) {
        const int r = idx / CH, c = idx % CH;
        if ((c >> 4) > (r >> 4)) sMm[r * LDC + c] = from_f32<Top>(0.f);
    }

    // ---- prefetch registers for phase 0 (row block w, channels l*CPT..) ----
    // Rows past the end of the sequence load the last valid row (always in
    // bounds) and are replaced by the padding values when unpacked.
    using RQ = RawRow<Tin, CPT>;
    using RA = RawRow<float, CPT>;
    typename RQ::T pq[16], pk[16];
    typename RA::T pa[16];
    float pbeta = 0.f;
    Tin pv[NJT][4];
    const int c0 = l * CPT;
    auto load_qka = [&](int ch) {
        const int base_r = ch * CH + w * 16;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = min(base_r + r, len - 1);
            const size_t off = ((size_t)(t0 + t) * H + h) * DK + c0;
            pq[r] = RQ::ld(gq + off);
            pk[r] = RQ::ld(gk + off);
            if (gate == 0) {
                if (!gl) {
                    pa[r] = RA::ld(ga + off);
                } else if constexpr (sizeof(Tin) == 4) {  // float32 logits, same layout
                    pa[r] = RA::ld(reinterpret_cast<const float*>(gg) + off);
                } else {  // bf16 logits, widened here
                    float x[CPT];
                    RQ::unpack(RQ::ld(gg + off), x);
                    pa[r] = RA::pack(x);
                }
            } else {  // one decay for every channel of the token, or none
                const size_t oh = (size_t)(t0 + t) * H + h;
                pa[r] = RA::splat(gate == 1 ? (gl ? to_f32(gg[oh]) : ga[oh]) : 1.f);
            }
        }
        if (w == 0) pbeta = gb[(size_t)(t0 + min(ch * CH + l, len - 1)) * H + h];
    };
    auto load_v = [&](int ch) {
#pragma unroll
        for (int jb = 0; jb < NJT; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = min(ch * CH + w * 16 + lg * 4 + e, len - 1);
                pv[jb][e] = gv[((size_t)(t0 + t) * H + h) * DV + col0 + jb * 16 + ln];
            }
    };

    const int nch = (len + CH - 1) / CH;
    if (nch > 0) { load_qka(0); load_v(0); }

    float pn_s[STW][4], pnm_s[STW][4];  // per owned state tile: Pn and Pn/Pm of its 4 rows
    bool bad = false;  // a chunk's decays left the chunk form's range (wave 0 checks)

    for (int ch = 0; ch < nch; ++ch) {
        // ================= phase 0a: running products inside row block w ======
        float pr[16][CPT];
        const int nvalid = len - (ch * CH + w * 16);  // valid rows of this row block
        {
            float run[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) run[c] = 1.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float a[CPT];
                RA::unpack(pa[r], a);
                if (gl) {
#pragma unroll
                    for (int c = 0; c < CPT; ++c) a[c] = sigmoid_f(a[c]);
                }
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    run[c] *= (r < nvalid) ? a[c] : 1.f;
                    pr[r][c] = run[c];
                }
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) sTot[w * DK + c0 + c] = run[c];
        }
        __syncthreads();  // B1

        // ================= phase 0b: decayed operands ==========================
        {
            // P_row / P_31 = (running product inside row block w) * fw with
            // fw = 1 / (t0 t1), 1 / t1, 1, t2 for w = 0..3 (t_b: row block b's
            // product), which forms no product over more than half a chunk
            float fw[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const float t0v = sTot[0 * DK + c0 + c], t1v = sTot[1 * DK + c0 + c];
                const float t2v = sTot[2 * DK + c0 + c], t3v = sTot[3 * DK + c0 + c];
                fw[c] = (w == 0) ? fast_rcp(t0v * t1v) : (w == 1) ? fast_rcp(t1v) : (w == 2) ? 1.f : t2v;
                if (w == 0 && gate != 2) bad |= decay_out_of_range(t0v * t1v, t2v * t3v);
            }
            Top kct[CPT][16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = w * 16 + r;
                float kx[CPT], qx[CPT];
                RQ::unpack(pk[r], kx);
                RQ::unpack(pq[r], qx);
                if (qn) {  // L2 norms of the row's k and q over the 64 lanes
                    float sk = 0.f, sq = 0.f;
#pragma unroll
                    for (int c = 0; c < CPT; ++c) { sk += kx[c] * kx[c]; sq += qx[c] * qx[c]; }
#pragma unroll
                    for (int off = 1; off < 64; off *= 2) {
                        sk += __shfl_xor(sk, off, 64);
                        sq += __shfl_xor(sq, off, 64);
                    }
                    const float ik = inv_norm(sk), iq = inv_norm(sq);
#pragma unroll
                    for (int c = 0; c < CPT; ++c) { kx[c] *= ik; qx[c] *= iq; }
                }
                Top kr[CPT], qr[CPT], kc[CPT];
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    const float kv = (r < nvalid) ? kx[c] : 0.f;
                    const float qv = (r < nvalid) ? qx[c] : 0.f;
                    const float ratio = pr[r][c] * fw[c];  // P_row / P_31
                    kr[c] = from_f32<Top>(kv * ratio);
                    qr[c] = from_f32<Top>(qv * ratio);
                    kc[c] = from_f32<Top>(kv * fast_rcp(ratio));
                    kct[c][r] = kc[c];
                }
                store_run<Top, CPT>(sKr + row * LDK + c0, kr);
                store_run<Top, CPT>(sQr + row * LDK + c0, qr);
                if (!L::KCT_ONLY) store_run<Top, CPT>(sKc + row * LDK + c0, kc);
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) store_run<Top, 16>(sKcT + (c0 + c) * LDC + w * 16, kct[c]);
            if (w == 0)
                sBeta[l] = (ch * CH + l < len)
                               ? ((p.fuse & FUSE_BETA_LOGITS) ? sigmoid_f(pbeta) : pbeta) : 0.f;
            // state operand SP = (Pm * S0)^T and the per-row decays kept for phase 4
#pragma unroll
            for (int i = 0; i < STW; ++i) {
                const int st = w + 4 * i;
                if (st < NST) {
                    const int ct = st / NJT_S, jj = st % NJT_S;
                    if (ckpt) {
                        float* cp = ckpt + ((size_t)(wi.t0 / CH + 2 * (long)seq + ch) * H + h) * DK * DV;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            cp[(size_t)(ct * 16 + lg * 4 + e) * DV + col0 + jj * 16 + ln] = S[i][e];
                    }
                    f32x4 sp;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = ct * 16 + lg * 4 + e;
                        const float a0 = sTot[c], a1 = sTot[DK + c];
                        const float a2 = sTot[2 * DK + c], a3 = sTot[3 * DK + c];
                        const float pm = a0 * a1;
                        pn_s[i][e] = pm * a2 * a3;
                        pnm_s[i][e] = a2 * a3;  // Pn / Pm
                        sp[e] = pm * S[i][e];
                    }
                    M::st4(sSP + (jj * 16 + ln) * LDK + ct * 16 + lg * 4, sp);
                }
            }
        }
        if (ch + 1 < nch) load_qka(ch + 1);
        __syncthreads();  // B2

        // ================= phase 1: Gram blocks, X and OI ======================
        f32x4 oi[NJT];
        {
            // Gram jobs (a, b), b <= a, dealt round-robin: wave w takes w, w+4, w+8.
            // Transposed tiles C' = Kc_b Kr_a^T give each lane 4 consecutive i of row r.
#pragma unroll
            for (int jn = w; jn < 10; jn += 4) {
                const int a = (jn >= 6) ? 3 : (jn >= 3) ? 2 : (jn >= 1) ? 1 : 0;
                const int b = jn - a * (a + 1) / 2;
                f32x4 cA = zero4(), cM = zero4();
#pragma unroll
                for (int s = 0; s < DK / 32; ++s) {
                    const auto fa = L::KCT_ONLY
                        ? gather32<Top>(sKcT + (s * 32 + lg * 8) * LDC + b * 16 + ln, LDC)
                        : M::ld32(sKc + (b * 16 + ln) * LDK + s * 32 + lg * 8);
                    const auto fk = M::ld32(sKr + (a * 16 + ln) * LDK + s * 32 + lg * 8);
                    const auto fq = M::ld32(sQr + (a * 16 + ln) * LDK + s * 32 + lg * 8);
                    cA = M::k32(fa, fk, cA);
                    cM = M::k32(fa, fq, cM);
                }
                // lane holds A[r = 16a + ln][i = 16b + 4lg + e], M likewise
                const int r = a * 16 + ln;
                const float br = sBeta[r];
                if (a == b) {
                    float4 ld;
                    ld.x = (lg * 4 + 0 < ln) ? br * cA[0] : 0.f;
                    ld.y = (lg * 4 + 1 < ln) ? br * cA[1] : 0.f;
                    ld.z = (lg * 4 + 2 < ln) ? br * cA[2] : 0.f;
                    ld.w = (lg * 4 + 3 < ln) ? br * cA[3] : 0.f;
                    *reinterpret_cast<float4*>(sLd + (a * 16 + ln) * L::LDL + lg * 4) = ld;
                    f32x4 mm;
#pragma unroll
                    for (int e = 0; e < 4; ++e) mm[e] = (lg * 4 + e <= ln) ? cM[e] : 0.f;
                    M::st4(sMm + r * LDC + b * 16 + lg * 4, mm);
                } else {
                    f32x4 lo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) lo[e] = br * cA[e];
                    M::st4(sLo + r * LDC + b * 16 + lg * 4, lo);
                    M::st4(sMm + r * LDC + b * 16 + lg * 4, cM);
                }
            }
            // X = V - Kr (Pm*S0) and OI = Qr (Pm*S0) for row block w
#pragma unroll
            for (int jb = 0; jb < NJT; ++jb) {
                f32x4 cx = zero4(), co = zero4();
#pragma unroll
                for (int s = 0; s < DK / 32; ++s) {
                    const auto fs = M::ld32(sSP + (jb * 16 + ln) * LDK + s * 32 + lg * 8);
                    const auto fk = M::ld32(sKr + (w * 16 + ln) * LDK + s * 32 + lg * 8);
                    const auto fq = M::ld32(sQr + (w * 16 + ln) * LDK + s * 32 + lg * 8);
                    cx = M::k32(fk, fs, cx);
                    co = M::k32(fq, fs, co);
                }
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = ch * CH + w * 16 + lg * 4 + e < len;
                    x[e] = (ok ? to_f32(pv[jb][e]) : 0.f) - cx[e];
                }
                M::st4(sX + (jb * 16 + ln) * LDC + w * 16 + lg * 4, x);
                oi[jb] = co;  // stays in registers until phase 4
            }
        }
        if (ch + 1 < nch) load_v(ch + 1);
        __syncthreads();  // B3

        // ================= phase 2: T = (I + Diag(beta) A)^{-1} Diag(beta) ====
        {
            // diagonal blocks: lane (block a = lg, column j = ln) solves L_aa x = e_j
            float x[16];
            const float* La = sLd + lg * 16 * L::LDL;
            float4 lrow[16][4];  // strictly lower part of the lane's block, issued at once
#pragma unroll
            for (int r = 1; r < 16; ++r)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    if (q4 * 4 < r) lrow[r][q4] = *reinterpret_cast<const float4*>(La + r * L::LDL + q4 * 4);
            // right-looking: once x[i] is final, remove it from every later row;
            // the updates of one step are independent of each other
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == ln) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < 15; ++i) {
#pragma unroll
                for (int r = i + 1; r < 16; ++r) {
                    const float4 v4 = lrow[r][i / 4];
                    const float lv = (i % 4 == 0) ? v4.x : (i % 4 == 1) ? v4.y : (i % 4 == 2) ? v4.z : v4.w;
                    x[r] -= lv * x[i];
                }
            }
            Top* Dr = sDr + (size_t)w * 4 * 16 * LDD;  // row-major copy, this wave only
            Top* Dc = sDc + (size_t)w * 4 * 16 * LDD;  // column-major copy
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

            // column block b = w: T_bb = D_b, T_ab = -D_a sum_{j=b}^{a-1} L_aj T_jb
            const int b = w;
            f32x4 TB[4];
            {
                // C-layout of D_b: lane holds rows 4lg..4lg+3 of column ln
#pragma unroll
                for (int e = 0; e < 4; ++e) TB[0][e] = to_f32(Dc[(b * 16 + ln) * LDD + lg * 4 + e]);
            }
            // TB[a - b] holds block (a, b)
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
            // write column block b of T = L^{-1} Diag(beta); zero above the diagonal
            const float bc = sBeta[b * 16 + ln];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int a = b + d;
                if (a < 4) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sTm[(a * 16 + lg * 4 + e) * LDC + b * 16 + ln] = from_f32<Top>(TB[d][e] * bc);
                }
            }
            for (int a = 0; a < b; ++a) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sTm[(a * 16 + lg * 4 + e) * LDC + b * 16 + ln] = from_f32<Top>(0.f);
            }
        }
        __syncthreads();  // B4

        // ================= phase 3: U = T X for row block w ====================
        {
            const int ns = (w >= 2) ? 2 : 1;
#pragma unroll
            for (int jb = 0; jb < NJT; ++jb) {
                f32x4 cu = zero4();
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s < ns) {
                        const auto ft = M::ld32(sTm + (w * 16 + ln) * LDC + s * 32 + lg * 8);
                        const auto fx = M::ld32(sX + (jb * 16 + ln) * LDC + s * 32 + lg * 8);
                        cu = M::k32(ft, fx, cu);
                    }
                }
                M::st4(sU + (jb * 16 + ln) * LDC + w * 16 + lg * 4, cu);
            }
        }
        __syncthreads();  // B5

        // ================= phase 4: outputs and the next state =================
        {
            const int ns = (w >= 2) ? 2 : 1;
#pragma unroll
            for (int jb = 0; jb < NJT; ++jb) {
                if (!go) break;
                f32x4 co = oi[jb];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s < ns) {
                        const auto fm = M::ld32(sMm + (w * 16 + ln) * LDC + s * 32 + lg * 8);
                        const auto fu = M::ld32(sU + (jb * 16 + ln) * LDC + s * 32 + lg * 8);
                        co = M::k32(fm, fu, co);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = ch * CH + w * 16 + lg * 4 + e;
                    if (t < len)
                        go[((size_t)(t0 + t) * H + h) * DV + col0 + jb * 16 + ln] =
                            from_f32<Tin>(p.scale * co[e]);
                }
            }
#pragma unroll
            for (int i = 0; i < STW; ++i) {
                const int st = w + 4 * i;
                if (st < NST) {
                    const int ct = st / NJT_S, jj = st % NJT_S;
                    f32x4 acc = zero4();
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const auto fk = M::ld32(sKcT + (ct * 16 + ln) * LDC + s * 32 + lg * 8);
                        const auto fu = M::ld32(sU + (jj * 16 + ln) * LDC + s * 32 + lg * 8);
                        acc = M::k32(fk, fu, acc);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[i][e] = pn_s[i][e] * S[i][e] + pnm_s[i][e] * acc[e];
                }
            }
        }
    }

    // ---- a work item with a chunk out of range is redone token by token ----
    {
        const uint64_t b = __builtin_amdgcn_ballot_w64(bad);
        __syncthreads();  // every wave is done with the last chunk's LDS
        if (l == 0) sBad[w] = b != 0;
        __syncthreads();
        if (sBad[0] | sBad[1] | sBad[2] | sBad[3]) {
            WalkArgs wa{};
            wa.q = p.q; wa.k = p.k; wa.v = p.v; wa.alpha = p.alpha; wa.beta = p.beta;
            wa.s0 = p.s0; wa.o = p.o; wa.sT = p.sT; wa.ckpt = ckpt;
            wa.H = H; wa.dv = DV; wa.gate = gate; wa.fuse = p.fuse; wa.scale = p.scale;
            __threadfence();  // this item's stores so far land before the walk's
            __syncthreads();
            token_walk<Tin, DK, DVT, NTH, false>(wa, seq, h, t0, len, col0, reinterpret_cast<float*>(smem));
            return;
        }
    }

    // ---- final state ----
    if (ckpt) {
        float* cp = ckpt + ((size_t)(wi.t0 / CH + 2 * (long)seq + nch) * H + h) * DK * DV;
#pragma unroll
        for (int i = 0; i < STW; ++i) {
            const int st = w + 4 * i;
            if (st < NST) {
                const int ct = st / NJT_S, jj = st % NJT_S;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    cp[(size_t)(ct * 16 + lg * 4 + e) * DV + col0 + jj * 16 + ln] = S[i][e];
            }
        }
    }
    if (p.sT) {
#pragma unroll
        for (int i = 0; i < STW; ++i) {
            const int st = w + 4 * i;
            if (st < NST) {
                const int ct = st / NJT_S, jj = st % NJT_S;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    p.sT[sbase + (size_t)(ct * 16 + lg * 4 + e) * DV + col0 + jj * 16 + ln] = S[i][e];
            }
        }
    }
}

// Longest-first order of the packed sequences (ties by index): rank by
// counting, one thread per sequence.  Quadratic in the number of sequences,
// which the host caps.
__global__ void order_sequences_kernel(const int* __restrict__ cu, int n, int* __restrict__ order) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int li = cu[i + 1] - cu[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) {
        const int lj = cu[j + 1] - cu[j];
        rank += (lj > li) || (lj == li && j < i);
    }
    order[rank] = i;
}

hipError_t launch_order_sequences(const int* cu_seqlens, int num_seqs, int* order,
                                  hipStream_t stream) {
    const int nb = (num_seqs + 255) / 256;
    hipLaunchKernelGGL(order_sequences_kernel, dim3(nb), dim3(256), 0, stream, cu_seqlens,
                       num_seqs, order);
    return hipGetLastError();
}

template <typename Tin, int DK, int DVT>
static hipError_t launch_chunk_t(const ChunkArgs& a, const int* order, hipStream_t stream) {
    using Lay = ChunkLayout<Tin, DK, DVT>;
    KParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.alpha = a.alpha; p.beta = a.beta; p.s0 = a.s0;
    p.o = a.o; p.sT = a.sT; p.cu_seqlens = a.cu_seqlens; p.order = order;
    const int nseq = a.cu_seqlens ? a.num_seqs : a.B;
    p.B = a.B; p.T = a.T; p.H = a.H; p.dv = a.dv;
    p.units = nseq * a.H;
    p.njt_all = a.dv / DVT;
    p.gate = a.gate;
    p.fuse = a.fuse;
    p.scale = a.scale;
    const int groups = (p.units + 7) / 8;
    const long grid = 8L * p.njt_all * groups;
    // once per instantiation (C++ guarantees a thread-safe initialisation)
    static const hipError_t attr = hipFuncSetAttribute(
        (const void*)chunk_fwd_kernel<Tin, DK, DVT>, hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((chunk_fwd_kernel<Tin, DK, DVT>), dim3((unsigned)grid), dim3(NTH),
                       Lay::bytes, stream, p, a.ckpt);
    return hipGetLastError();
}

template <typename Tin, int DK>
static hipError_t launch_chunk_dk(const ChunkArgs& a, int dvt, const int* order,
                                  hipStream_t stream) {
    if constexpr (sizeof(Tin) == 4 && DK == 128) {
        // fp32 operands at dk = 128 only fit in LDS with 16-column slices
        (void)dvt;
        return launch_chunk_t<Tin, DK, 16>(a, order, stream);
    } else {
        switch (dvt) {
            case 16: return launch_chunk_t<Tin, DK, 16>(a, order, stream);
            case 32: return launch_chunk_t<Tin, DK, 32>(a, order, stream);
            default: return launch_chunk_t<Tin, DK, 64>(a, order, stream);
        }
    }
}

int plan_chunk_dvt(int units, int dv, bool bf16) {
    // widest value tile that still gives every compute unit a workgroup
    (void)bf16;
    for (int dvt = 64; dvt >= 16; dvt /= 2)
        if (dvt <= dv && (long)units * (dv / dvt) >= 256) return dvt;
    return 16;
}

hipError_t launch_chunk_fwd(const ChunkArgs& a, hipStream_t stream) {
    const int nseq = a.cu_seqlens ? a.num_seqs : a.B;
    const int units = nseq * a.H;
    if (units == 0) return hipSuccess;
    if (a.split_ws) return launch_chunk_split(a, a.split_ws, stream);
    const int* order = nullptr;
    if (a.cu_seqlens && a.order) {
        hipError_t e = launch_order_sequences(a.cu_seqlens, a.num_seqs, a.order, stream);
        if (e != hipSuccess) return e;
        order = a.order;
    }
    int dvt = a.dvt > 0 ? a.dvt : plan_chunk_dvt(units, a.dv, a.bf16);
    if (dvt > a.dv) dvt = a.dv;
    if (a.bf16 && !a.generic && chunk_bf16_supports(dvt)) {
        KParams p;
        p.q = a.q; p.k = a.k; p.v = a.v; p.alpha = a.alpha; p.beta = a.beta; p.s0 = a.s0;
        p.o = a.o; p.sT = a.sT; p.cu_seqlens = a.cu_seqlens; p.order = order;
        p.B = a.B; p.T = a.T; p.H = a.H; p.dv = a.dv;
        p.units = units;
        p.njt_all = a.dv / dvt;
        p.gate = a.gate;
        p.fuse = a.fuse;
        p.scale = a.scale;
        p.ckpt = a.ckpt;
        return launch_chunk_bf16(p, a.dk, dvt, stream);
    }
    if (a.bf16)
        return a.dk == 128 ? launch_chunk_dk<bf16_t, 128>(a, dvt, order, stream)
                           : launch_chunk_dk<bf16_t, 64>(a, dvt, order, stream);
    return a.dk == 128 ? launch_chunk_dk<float, 128>(a, dvt, order, stream)
                       : launch_chunk_dk<float, 64>(a, dvt, order, stream);
}

// ---------------------------------------------------------------------------
// The scratch of kda_chunk_fwd_noalloc: the longest-first order of the packed
// sequences (written in full by order_sequences_kernel before each use, so it
// needs no clearing) lives in this file-scope device array instead of a
// caller workspace.  Each GPU the library runs on holds its own copy, at its
// own address, until the process ends.  In host code the array's name is only
// a host-side stand-in: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
static __device__ __align__(256) int scratch[NOALLOC_MAX_SEQS];

hipError_t noalloc_order_buffer(hipStream_t stream, int** out) {
    constexpr int kMaxDevices = 64;
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = static_cast<int*>(addr[dev]);
    return hipSuccess;
}

}  // namespace kda
