// gdn2_chunk.hip -- chunk-wise Gated DeltaNet-2 forward on gfx950 matrix cores.
//
// Method: "线性注意力机制：从标准注意力到 Gated DeltaNet-2" (jindou-blog),
// section 4 "Gated DeltaNet-2：解耦擦除与写入", read as the KDA step with the
// delta rule's write strength split into an erase gate e_t and a write gate
// w_t per key channel (row of S):
//     S_t = S~ - a_t (S~^T k_t)^T + c_t v_t^T,   S~ = Diag(alpha_t) S_{t-1},
//     a_t = e_t . k_t,  c_t = w_t . k_t,         o_t = scale S_t^T q_t,
// computed in the chunk-wise mode of bugfactory.tech news 3610, fifth
// paragraph (matrix products inside a chunk, the state carried between
// chunks; the kongchang.com page, section "硬件效率的优化策略").  The chunk
// identities follow from the update (the pages print none).  For a chunk of
// C = 64 tokens from state S0 with P_r the running product of alpha up to
// token r, write Kbar = K*P, A~ = A/P, C~ = C/P (rows scaled per channel) and
// let p_r = S~_r^T k_r be the predictions.  Unrolling the chunk gives
//     (I + L_a) Pred = Kbar S0 + L_c V,   L_a = tril_-1(Kbar A~^T), L_c = tril_-1(Kbar C~^T)
//     O   = scale (Qbar S0 + M_c V - M_a Pred),  M_* = tril(Qbar *~^T)
//     S_C = Diag(P_63) (S0 + C~^T V - A~^T Pred).
// Each token writes two rows (c_r with v_r, a_r with -p_r), so the output and
// the state update are 128-deep products over the stacked rows F = [C~; A~]
// and Z = [V; -Pred].  As in the KDA kernels, decays are referenced to the
// middle of the chunk (Pm = P_31) so that both factors of every Gram product
// span alpha's product over half a chunk only (a chunk where that product
// falls below 2^-100 in some channel sends its work item to the exact token
// walk of chunk_walk.h):
//     Kr = K*P/Pm, Qr = Q*P/Pm, Ec = (e.K)*Pm/P, Wc = (w.K)*Pm/P,  SP = Pm*S0
//     Y = Kr SP + tril_-1(Kr Wc^T) V,  Pred = (I + tril_-1(Kr Ec^T))^{-1} Y
//     O = scale (Qr SP + [tril(Qr Wc^T) | tril(Qr Ec^T)] Z)
//     S_C = Pn*S0 + (Pn/Pm) * ([Wc; Ec]^T Z)
// Past the end of a sequence the chunk is padded with q = k = v = 0,
// e = w = 0, alpha = 1, an exact no-op.
//
// Work decomposition as in the KDA kernels: one workgroup owns one (unit,
// value-column slice) and walks the unit's chunks with its fp32 state slice
// in matrix-core accumulator registers; the column-independent work (decays,
// Gram products, the triangular inverse) is recomputed per slice, and the
// slices of a unit share an XCD.  A chunk runs in five phases separated by
// workgroup barriers (decays; operands; Gram products and Kr SP, Qr SP; Y and
// the inverse; the solve; outputs and the state update), with the next
// chunk's inputs loaded into registers one chunk ahead.  Wave w works on row
// block w mod 4 of the chunk.  With dk = 128 and 32-column slices the
// workgroup has eight waves, two per SIMD: the two waves of a row block split
// its rows in the operand build and its two value tiles in the products, and
// each holds two state tiles; the phases are chains of dependent matrix-core
// products and LDS round trips, which the second wave on a SIMD overlaps.
// There the diagonal blocks of L_a are inverted in the Gram phase, each by
// the wave that formed it, while the other four waves take the rest of the
// Gram blocks.  Other shapes run four waves.
#include "chunk_walk.h"

namespace kda {

namespace {


struct G2Params {
    KParams base;                // q, k, v, alpha (NULL: no forget gate), s0, o, sT, mapping
    const float *erase, *write;  // [tokens, H, dk]
};

template <int DK, int DVT>
struct G2Layout {
    static constexpr int ES = 2;                  // bf16 operands
    static constexpr int LDK = DK + 8;            // [token][channel] tiles
    static constexpr int LDC = CH + 8;            // [*][token] tiles
    static constexpr int LDC2 = 2 * CH + 8;       // [*][stacked row] tiles
    static constexpr int LDD = 16 + 8;            // 16x16 blocks
    static constexpr int LDL = 20;                // fp32 diagonal blocks of L_a
    static constexpr int NJT = DVT / 16;
    static constexpr int NCT = DK / 16;
    static constexpr int NST = NCT * NJT;
    // region A, phases 0b-1: chunk operands
    static constexpr size_t oKr = 0;
    static constexpr size_t oQr = oKr + (size_t)CH * LDK * ES;
    static constexpr size_t oEc = oQr + (size_t)CH * LDK * ES;
    static constexpr size_t oWc = oEc + (size_t)CH * LDK * ES;
    static constexpr size_t oSP = oWc + (size_t)CH * LDK * ES;
    static constexpr size_t endA1 = oSP + (size_t)DVT * LDK * ES;
    // region A, phases 1b-3 (overlays the above)
    static constexpr size_t oTm = 0;
    static constexpr size_t oYT = oTm + (size_t)CH * LDC * ES;
    static constexpr size_t oDr = oYT + (size_t)DVT * LDC * ES;
    static constexpr size_t oDc = oDr + (size_t)4 * 4 * 16 * LDD * ES;
    static constexpr size_t endA2 = oDc + (size_t)4 * 4 * 16 * LDD * ES;
    static constexpr size_t endA = endA1 > endA2 ? endA1 : endA2;
    // region B
    static constexpr size_t oFT = (endA + 255) / 256 * 256;        // [DK][LDC2]: [Wc; Ec]^T
    static constexpr size_t oM = oFT + (size_t)DK * LDC2 * ES;     // [CH][LDC2]: [M_c | M_a]
    static constexpr size_t oZT = oM + (size_t)CH * LDC2 * ES;     // [DVT][LDC2]: [V; -Pred]^T
    static constexpr size_t oAc = oZT + (size_t)DVT * LDC2 * ES;   // [CH][LDC]: L_c
    static constexpr size_t oLo = oAc + (size_t)CH * LDC * ES;     // [CH][LDC]: L_a off-diagonal
    static constexpr size_t oLd = oLo + (size_t)CH * LDC * ES;     // fp32 [4][16][LDL]
    static constexpr size_t oBad = oLd + (size_t)4 * 16 * LDL * 4;   // u32 [8] out-of-range flags
    static constexpr size_t bytes = oBad + 32;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// CPT = DK/64 consecutive channels of one token row in their stored form
template <int CPT> struct G2Row;
template <> struct G2Row<1> {
    typedef uint16_t B;  // bf16
    typedef float F;
    static __device__ __forceinline__ B ldb(const bf16_t* p) { return *reinterpret_cast<const uint16_t*>(p); }
    static __device__ __forceinline__ F ldf(const float* p) { return *p; }
    static __device__ __forceinline__ void ub(B w, float* x) { x[0] = __uint_as_float(uint32_t(w) << 16); }
    static __device__ __forceinline__ void uf(F w, float* x) { x[0] = w; }
    static __device__ __forceinline__ F one() { return 1.f; }
};
template <> struct G2Row<2> {
    typedef uint32_t B;
    typedef float2 F;
    static __device__ __forceinline__ B ldb(const bf16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
    static __device__ __forceinline__ F ldf(const float* p) { return *reinterpret_cast<const float2*>(p); }
    static __device__ __forceinline__ void ub(B w, float* x) {
        x[0] = __uint_as_float(w << 16);
        x[1] = __uint_as_float(w & 0xffff0000u);
    }
    static __device__ __forceinline__ void uf(F w, float* x) { x[0] = w.x; x[1] = w.y; }
    static __device__ __forceinline__ F one() { return make_float2(1.f, 1.f); }
};

// x = (I + L)^{-1} e_j for a strictly lower triangular 16x16 block L stored
// by columns (column i: rows 0..15 at Lc + i ld, 16-byte aligned), by forward
// substitution one column of L at a time
__device__ __forceinline__ void unit_lower_solve(const float* Lc, int ld, int j, float (&x)[16]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
    for (int i = 0; i < 15; ++i) {
        float col[16];
#pragma unroll
        for (int q4 = (i + 1) / 4; q4 < 4; ++q4) {
            const float4 v4 = *reinterpret_cast<const float4*>(Lc + i * ld + q4 * 4);
            col[q4 * 4] = v4.x; col[q4 * 4 + 1] = v4.y; col[q4 * 4 + 2] = v4.z; col[q4 * 4 + 3] = v4.w;
        }
#pragma unroll
        for (int r = i + 1; r < 16; ++r) x[r] -= col[r] * x[i];
    }
}

template <int DK, int DVT, int NW>
__global__ __launch_bounds__(NW * 64, 1) void gdn2_chunk_kernel(G2Params gp) {
    using Top = bf16_t;
    using L = G2Layout<DK, DVT>;
    using M = Mma<Top>;
    constexpr int NTH = NW * 64;
    constexpr int NH = NW / 4;          // waves per row block
    constexpr int NSB = 4 * NH;         // operand-build row blocks, one per wave
    constexpr int RPW = CH / NSB;       // rows of a wave's operand build
    constexpr int CPT = DK / 64;        // channels per lane in a row
    constexpr int LDK = L::LDK, LDC = L::LDC, LDC2 = L::LDC2, LDD = L::LDD, NJT = L::NJT;
    constexpr int NJW = NJT / NH;       // value tiles per wave
    constexpr int NST = L::NST, STW = (NST + NW - 1) / NW;
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    static_assert(CPT >= 1 && NJW >= 1 && RPW % 4 == 0, "a wave's share of a row block");
    using R = G2Row<CPT>;
    const KParams& p = gp.base;

    extern __shared__ __align__(16) unsigned char smem[];
    Top* sKr = reinterpret_cast<Top*>(smem + L::oKr);
    Top* sQr = reinterpret_cast<Top*>(smem + L::oQr);
    Top* sEc = reinterpret_cast<Top*>(smem + L::oEc);
    Top* sWc = reinterpret_cast<Top*>(smem + L::oWc);
    Top* sSP = reinterpret_cast<Top*>(smem + L::oSP);
    Top* sTm = reinterpret_cast<Top*>(smem + L::oTm);
    Top* sYT = reinterpret_cast<Top*>(smem + L::oYT);
    Top* sDr = reinterpret_cast<Top*>(smem + L::oDr);
    Top* sDc = reinterpret_cast<Top*>(smem + L::oDc);
    Top* sFT = reinterpret_cast<Top*>(smem + L::oFT);
    Top* sM = reinterpret_cast<Top*>(smem + L::oM);
    Top* sZT = reinterpret_cast<Top*>(smem + L::oZT);
    Top* sAc = reinterpret_cast<Top*>(smem + L::oAc);
    Top* sLo = reinterpret_cast<Top*>(smem + L::oLo);
    float* sLd = reinterpret_cast<float*>(smem + L::oLd);
    uint32_t* sBad = reinterpret_cast<uint32_t*>(smem + L::oBad);
    static_assert(WalkShape<DVT, NTH, true>::lds_bytes <= L::oBad, "walk LDS");
    // the decay totals of the operand-build row blocks (phases 0a-0b) share
    // the LDS of L_a's diagonal blocks (phases 1-2)
    static_assert((size_t)NSB * DK * 4 <= (size_t)4 * 16 * L::LDL * 4, "decay totals");
    auto tot = [&](int b, int c) -> float& { return sLd[b * DK + c]; };
    // [row][channel] tiles at dk = 128: the 16-byte chunk c of row r sits at
    // chunk (c + 7 (r mod 2)) mod 16, which spreads fragment reads of 16 rows
    // over all LDS banks (the plain 272-byte rows pair them two by two)
    auto tk = [&](int row, int ch) -> int {
        if constexpr (DK == 128) return row * LDK + ((((ch >> 3) + 7 * (row & 1)) & 15) << 3) + (ch & 7);
        else return row * LDK + ch;
    };

    const WorkItem wi = decode_work(p);
    if (!wi.valid) return;
    const int H = p.H, h = wi.h, seq = wi.seq, jt = wi.jt, len = wi.len;
    const long t0 = wi.t0;
    const int DV = p.dv;
    const bf16_t* __restrict__ gq = static_cast<const bf16_t*>(p.q);
    const bf16_t* __restrict__ gk = static_cast<const bf16_t*>(p.k);
    const bf16_t* __restrict__ gv = static_cast<const bf16_t*>(p.v);
    const float* __restrict__ ga = static_cast<const float*>(p.alpha);
    const float* __restrict__ ge = gp.erase;
    const float* __restrict__ gw = gp.write;
    // Every load of the chunk loop is issued on every path (a load under a
    // branch would make the compiler's waits for the loads in flight assume
    // the path without it, and wait for more): without a forget gate the
    // decay rows are read from the erase gate, an array of the same shape,
    // and replaced by 1 where they are used.
    const bool has_alpha = ga != nullptr;
    const float* __restrict__ gsa = has_alpha ? ga : ge;
    bf16_t* __restrict__ go = static_cast<bf16_t*>(p.o);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rb = w & 3;        // row block of the wave's products
    const int hf = w >> 2;       // its share of them: value tiles hf*NJW..
    const int jb0 = hf * NJW;
    const int sb = rb * NH + hf; // operand build: rows sb*RPW .. sb*RPW + RPW - 1
    const int l = tid & 63;
    const int ln = l & 15;
    const int lg = l >> 4;
    const int col0 = jt * DVT;

    // ---- state slice in C-layout registers: wave w owns tiles w, w+NW, ... ----
    f32x4 S[STW];
    const size_t sbase = ((size_t)seq * H + h) * DK * DV;
#pragma unroll
    for (int i = 0; i < STW; ++i) {
        const int st = w + NW * i;
        S[i] = zero4();
        if (st < NST && p.s0) {
            const int ct = st / NJT, jj = st % NJT;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[i][e] = p.s0[sbase + (size_t)(ct * 16 + lg * 4 + e) * DV + col0 + jj * 16 + ln];
        }
    }

    // Blocks above the diagonal of M (both halves) and of L_c are read by the
    // 32-deep steps and must be zero; nothing else writes them.
    for (int idx = tid; idx < CH * 2 * CH; idx += NTH) {
        const int r = idx / (2 * CH), c = idx % (2 * CH);
        if (((c & (CH - 1)) >> 4) > (r >> 4)) sM[r * LDC2 + c] = from_f32<Top>(0.f);
    }
    for (int idx = tid; idx < CH * CH; idx += NTH) {
        const int r = idx / CH, c = idx % CH;
        if ((c >> 4) > (r >> 4)) sAc[r * LDC + c] = from_f32<Top>(0.f);
    }

    // ---- register prefetch: rows of block sb, channels c0..; V of row block rb ----
    typename R::B pq[RPW], pk[RPW];
    typename R::F pa[RPW], pe[RPW], pw[RPW];
    bf16_t pv[NJW][4];
    const int c0 = l * CPT;
    // a quarter of the rows per part: the loads of the next chunk go
    // out in four parts, at the end of the operand build and after each of the
    // barriers B2..B4, where they overlap matrix-core work instead of stalling
    // the operand build on their issue (80 load instructions per lane and chunk)
    auto load_rows = [&](int ch, int part) {
        const int base_r = ch * CH + sb * RPW;
#pragma unroll
        for (int r = part * RPW / 4; r < (part + 1) * RPW / 4; ++r) {
            const int t = min(base_r + r, len - 1);  // rows past the end are replaced when used
            const size_t off = ((size_t)(t0 + t) * H + h) * DK + c0;
            pq[r] = R::ldb(gq + off);
            pk[r] = R::ldb(gk + off);
            pa[r] = R::ldf(gsa + off);
            pe[r] = R::ldf(ge + off);
            pw[r] = R::ldf(gw + off);
        }
    };
    auto load_v = [&](int ch) {
#pragma unroll
        for (int jj = 0; jj < NJW; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = min(ch * CH + rb * 16 + lg * 4 + e, len - 1);
                pv[jj][e] = gv[((size_t)(t0 + t) * H + h) * DV + col0 + (jb0 + jj) * 16 + ln];
            }
    };

    const int nch = (len + CH - 1) / CH;
    if (nch > 0) {
#pragma unroll
        for (int part = 0; part < 4; ++part) load_rows(0, part);
        load_v(0);
    }

    float pn_s[STW][4], pnm_s[STW][4];
    bool bad = false;  // a chunk's decays left the chunk form's range (wave 0 checks)

    for (int ch = 0; ch < nch; ++ch) {
        // ================= phase 0a: running products inside row block sb =====
        float pr[RPW][CPT];
        const int nvalid = len - (ch * CH + sb * RPW);
        {
            float run[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) run[c] = 1.f;
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                float a[CPT];
                R::uf(pa[r], a);
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    run[c] *= (r < nvalid && has_alpha) ? a[c] : 1.f;
                    pr[r][c] = run[c];
                }
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) tot(sb, c0 + c) = run[c];
        }
        __syncthreads();  // B1

        // ================= phase 0b: decayed operands ==========================
        {
            // P_row / P_31 = (running product inside row block sb) * fw with
            // fw = 1 / (t_sb ... t_{h-1}) below the middle h = NSB/2 and
            // t_h ... t_{sb-1} from it on (t_b: row block b's product): no
            // product over more than half a chunk is formed
            // lo = Pm = P_31 and hi = Pn / Pm of the lane's channels
            float fw[CPT], lo[CPT], hi[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                float f = 1.f;
                lo[c] = 1.f;
                hi[c] = 1.f;
#pragma unroll
                for (int b = 0; b < NSB / 2; ++b) {
                    lo[c] *= tot(b, c0 + c);
                    hi[c] *= tot(NSB / 2 + b, c0 + c);
                }
                if (sb < NSB / 2) {
                    for (int b = sb; b < NSB / 2; ++b) f *= tot(b, c0 + c);
                    f = fast_rcp(f);
                } else {
                    for (int b = NSB / 2; b < sb; ++b) f *= tot(b, c0 + c);
                }
                fw[c] = f;
                if (sb == 0) bad |= decay_out_of_range(lo[c], hi[c]);
            }
            Top wct[CPT][RPW], ect[CPT][RPW];
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const int row = sb * RPW + r;
                const bool ok = r < nvalid;
                float kx[CPT], qx[CPT], ex[CPT], wx[CPT];
                R::ub(pk[r], kx);
                R::ub(pq[r], qx);
                R::uf(pe[r], ex);
                R::uf(pw[r], wx);
                Top kr[CPT], qr[CPT], ec[CPT], wc[CPT];
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    const float kv = ok ? kx[c] : 0.f;
                    const float qv = ok ? qx[c] : 0.f;
                    const float ratio = pr[r][c] * fw[c];  // P_row / P_31
                    const float inv = fast_rcp(ratio);
                    kr[c] = from_f32<Top>(kv * ratio);
                    qr[c] = from_f32<Top>(qv * ratio);
                    ec[c] = from_f32<Top>(ex[c] * kv * inv);
                    wc[c] = from_f32<Top>(wx[c] * kv * inv);
                    ect[c][r] = ec[c];
                    wct[c][r] = wc[c];
                }
                store_run<Top, CPT>(sKr + tk(row, c0), kr);
                store_run<Top, CPT>(sQr + tk(row, c0), qr);
                store_run<Top, CPT>(sEc + tk(row, c0), ec);
                store_run<Top, CPT>(sWc + tk(row, c0), wc);
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                store_run<Top, RPW>(sFT + (c0 + c) * LDC2 + sb * RPW, wct[c]);
                store_run<Top, RPW>(sFT + (c0 + c) * LDC2 + CH + sb * RPW, ect[c]);
            }
            // V^T into the first half of Z (4 consecutive tokens per lane)
#pragma unroll
            for (int jj = 0; jj < NJW; ++jj) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x[e] = (ch * CH + rb * 16 + lg * 4 + e < len) ? to_f32(pv[jj][e]) : 0.f;
                M::st4(sZT + ((jb0 + jj) * 16 + ln) * LDC2 + rb * 16 + lg * 4, x);
            }
            // SP = (Pm * S0)^T and the per-row decays kept for the state update
            // (Pm and Pn / Pm of channel c come from lane c / CPT)
#pragma unroll
            for (int i = 0; i < STW; ++i) {
                const int st = w + NW * i;
                if (st < NST) {
                    const int ct = st / NJT, jj = st % NJT;
                    f32x4 sp;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int src = (ct * 16 + lg * 4 + e) / CPT;
                        const float pm = __shfl(lo[e % CPT], src, 64);
                        const float pnm = __shfl(hi[e % CPT], src, 64);
                        pn_s[i][e] = pm * pnm;
                        pnm_s[i][e] = pnm;  // Pn / Pm
                        sp[e] = pm * S[i][e];
                    }
                    M::st4(sSP + tk(jj * 16 + ln, ct * 16 + lg * 4), sp);
                }
            }
        }
        load_rows(ch + 1, 0);  // (past the last chunk: rows clamped to the last, unused)
        __syncthreads();  // B2
        load_rows(ch + 1, 1);

        // ================= phase 1: Gram blocks, X = Kr SP and OI = Qr SP =====
        f32x4 xr[NJW], oi[NJW];
        {
            // Gram jobs (a, b), b <= a; transposed tiles F_b Kr_a^T give each
            // lane 4 consecutive i of row r = 16a + ln.  A job forms the L part
            // (L_a, L_c from Kr) and the M part (M_a, M_c from Qr), or one of them.
            auto gram = [&](int jn, bool doL, bool doM) {
                const int a = (jn >= 6) ? 3 : (jn >= 3) ? 2 : (jn >= 1) ? 1 : 0;
                const int b = jn - a * (a + 1) / 2;
                f32x4 cLa = zero4(), cLc = zero4(), cMa = zero4(), cMc = zero4();
#pragma unroll
                for (int s = 0; s < DK / 32; ++s) {
                    const auto fe = M::ld32(sEc + tk(b * 16 + ln, s * 32 + lg * 8));
                    const auto fw = M::ld32(sWc + tk(b * 16 + ln, s * 32 + lg * 8));
                    if (doL) {
                        const auto fk = M::ld32(sKr + tk(a * 16 + ln, s * 32 + lg * 8));
                        cLa = M::k32(fe, fk, cLa);
                        cLc = M::k32(fw, fk, cLc);
                    }
                    if (doM) {
                        const auto fq = M::ld32(sQr + tk(a * 16 + ln, s * 32 + lg * 8));
                        cMa = M::k32(fe, fq, cMa);
                        cMc = M::k32(fw, fq, cMc);
                    }
                }
                const int r = a * 16 + ln;
                if (a == b) {
                    if (doL) {
                        // the diagonal block, strictly lower, stored by columns
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sLd[(a * 16 + lg * 4 + e) * L::LDL + ln] = (lg * 4 + e < ln) ? cLa[e] : 0.f;
                        f32x4 lc;
#pragma unroll
                        for (int e = 0; e < 4; ++e) lc[e] = (lg * 4 + e < ln) ? cLc[e] : 0.f;
                        M::st4(sAc + r * LDC + b * 16 + lg * 4, lc);
                    }
                    if (doM) {
                        f32x4 mc, ma;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            mc[e] = (lg * 4 + e <= ln) ? cMc[e] : 0.f;
                            ma[e] = (lg * 4 + e <= ln) ? cMa[e] : 0.f;
                        }
                        M::st4(sM + r * LDC2 + b * 16 + lg * 4, mc);
                        M::st4(sM + r * LDC2 + CH + b * 16 + lg * 4, ma);
                    }
                } else {
                    if (doL) {
                        M::st4(sLo + r * LDC + b * 16 + lg * 4, cLa);
                        M::st4(sAc + r * LDC + b * 16 + lg * 4, cLc);
                    }
                    if (doM) {
                        M::st4(sM + r * LDC2 + b * 16 + lg * 4, cMc);
                        M::st4(sM + r * LDC2 + CH + b * 16 + lg * 4, cMa);
                    }
                }
            };
            if constexpr (NW == 8) {
                if (hf == 0) {
                    // the L part of diagonal block rb, then its inverse
                    // D = (I + L_aa)^{-1} (lane (ln, any lg) forms column ln),
                    // which replaces L_aa in LDS, by columns
                    gram(rb * (rb + 3) / 2, true, false);
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    float* La = sLd + rb * 16 * L::LDL;
                    float x[16];
                    unit_lower_solve(La, L::LDL, ln, x);
                    if (lg == 0) {
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4)
                            *reinterpret_cast<float4*>(La + ln * L::LDL + r4 * 4) =
                                make_float4(x[r4 * 4], x[r4 * 4 + 1], x[r4 * 4 + 2], x[r4 * 4 + 3]);
                    }
                } else {
                    // the six off-diagonal jobs: (1,0) or (2,0) or (2,1) or
                    // (3,0) whole, and half of (3,2) or (3,1); and the M part
                    // of diagonal block rb
                    gram(rb == 0 ? 1 : rb == 1 ? 3 : rb == 2 ? 4 : 6, true, true);
                    gram(rb < 2 ? 8 : 7, (rb & 1) == 0, (rb & 1) != 0);
                    gram(rb * (rb + 3) / 2, false, true);
                }
            } else {
#pragma unroll
                for (int jn = w; jn < 10; jn += NW) gram(jn, true, true);
            }
#pragma unroll
            for (int jj = 0; jj < NJW; ++jj) {
                const int jb = jb0 + jj;
                f32x4 cx = zero4(), co = zero4();
#pragma unroll
                for (int s = 0; s < DK / 32; ++s) {
                    const auto fs = M::ld32(sSP + tk(jb * 16 + ln, s * 32 + lg * 8));
                    const auto fk = M::ld32(sKr + tk(rb * 16 + ln, s * 32 + lg * 8));
                    const auto fq = M::ld32(sQr + tk(rb * 16 + ln, s * 32 + lg * 8));
                    cx = M::k32(fk, fs, cx);
                    co = M::k32(fq, fs, co);
                }
                xr[jj] = cx;
                oi[jj] = co;
            }
        }
        load_v(ch + 1);
        __syncthreads();  // B3
        load_rows(ch + 1, 2);

        // ================= phase 2: Y = X + L_c V, T = (I + L_a)^{-1} ===========
        {
            const int ns = (rb >= 2) ? 2 : 1;
#pragma unroll
            for (int jj = 0; jj < NJW; ++jj) {
                const int jb = jb0 + jj;
                f32x4 cy = xr[jj];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s < ns) {
                        const auto fa = M::ld32(sAc + (rb * 16 + ln) * LDC + s * 32 + lg * 8);
                        const auto fv = M::ld32(sZT + (jb * 16 + ln) * LDC2 + s * 32 + lg * 8);
                        cy = M::k32(fa, fv, cy);
                    }
                }
                M::st4(sYT + (jb * 16 + ln) * LDC + rb * 16 + lg * 4, cy);
            }
            if constexpr (NW == 8) {
                // the first four waves form T's column blocks from the
                // inverses D_a left in LDS by columns (rounded to the operand
                // type where they are used)
                if (hf == 0) {
                    const int b = rb;
                    f32x4 TB[4];
                    {
                        const float4 d4 = *reinterpret_cast<const float4*>(sLd + (b * 16 + ln) * L::LDL + lg * 4);
                        TB[0][0] = to_f32(from_f32<Top>(d4.x)); TB[0][1] = to_f32(from_f32<Top>(d4.y));
                        TB[0][2] = to_f32(from_f32<Top>(d4.z)); TB[0][3] = to_f32(from_f32<Top>(d4.w));
                    }
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
                            f32x4 dr;
#pragma unroll
                            for (int e = 0; e < 4; ++e) dr[e] = sLd[(a * 16 + lg * 4 + e) * L::LDL + ln];
                            f32x4 t = M::k16(M::pack16(dr), M::pack16(y), zero4());
                            TB[d][0] = -t[0]; TB[d][1] = -t[1]; TB[d][2] = -t[2]; TB[d][3] = -t[3];
                        }
                    }
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const int a = b + d;
                        if (a < 4) {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                sTm[(a * 16 + lg * 4 + e) * LDC + b * 16 + ln] = from_f32<Top>(TB[d][e]);
                        }
                    }
                    for (int a = 0; a < b; ++a) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sTm[(a * 16 + lg * 4 + e) * LDC + b * 16 + ln] = from_f32<Top>(0.f);
                    }
                }
            } else {
                // the first four waves form T's column blocks
                if (hf == 0) {
                    // diagonal blocks: lane (block lg, column ln) forms column ln
                    // of D_lg = (I + L_aa)^{-1}
                    float x[16];
                    unit_lower_solve(sLd + lg * 16 * L::LDL, L::LDL, ln, x);
                    Top* Dr = sDr + (size_t)rb * 4 * 16 * LDD;
                    Top* Dc = sDc + (size_t)rb * 4 * 16 * LDD;
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

                    // column block b = rb: T_bb = D_b, T_ab = -D_a sum_{j=b}^{a-1} L_aj T_jb
                    const int b = rb;
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
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const int a = b + d;
                        if (a < 4) {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                sTm[(a * 16 + lg * 4 + e) * LDC + b * 16 + ln] = from_f32<Top>(TB[d][e]);
                        }
                    }
                    for (int a = 0; a < b; ++a) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sTm[(a * 16 + lg * 4 + e) * LDC + b * 16 + ln] = from_f32<Top>(0.f);
                    }
                }
            }
        }
        __syncthreads();  // B4
        load_rows(ch + 1, 3);

        // ================= phase 3: Pred = T Y, stored as -Pred^T in Z ==========
        {
            const int ns = (rb >= 2) ? 2 : 1;
#pragma unroll
            for (int jj = 0; jj < NJW; ++jj) {
                const int jb = jb0 + jj;
                f32x4 cp = zero4();
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s < ns) {
                        const auto ft = M::ld32(sTm + (rb * 16 + ln) * LDC + s * 32 + lg * 8);
                        const auto fy = M::ld32(sYT + (jb * 16 + ln) * LDC + s * 32 + lg * 8);
                        cp = M::k32(ft, fy, cp);
                    }
                }
                f32x4 np = {-cp[0], -cp[1], -cp[2], -cp[3]};
                M::st4(sZT + (jb * 16 + ln) * LDC2 + CH + rb * 16 + lg * 4, np);
            }
        }
        __syncthreads();  // B5

        // ================= phase 4: outputs and the next state =================
        {
            const int ns = (rb >= 2) ? 2 : 1;
            const Rsrc ro = make_rsrc(go + ((size_t)(t0 + (long)ch * CH) * H + h) * DV,
                                      (uint32_t)(min(len - ch * CH, CH) * H * DV * 2));
#pragma unroll
            for (int jj = 0; jj < NJW; ++jj) {
                const int jb = jb0 + jj;
                f32x4 co = oi[jj];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        if (s < ns) {
                            const int k0 = half * CH + s * 32 + lg * 8;
                            const auto fm = M::ld32(sM + (rb * 16 + ln) * LDC2 + k0);
                            const auto fz = M::ld32(sZT + (jb * 16 + ln) * LDC2 + k0);
                            co = M::k32(fm, fz, co);
                        }
                    }
                }
                // rows past the end of the sequence lie outside the descriptor
                // (lane part: row 16rb + 4lg, column col0 + ln; wave part: row e,
                // column tile jb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    __builtin_amdgcn_raw_buffer_store_b16(
                        __builtin_bit_cast(unsigned short, from_f32<bf16_t>(p.scale * co[e])), ro,
                        (uint32_t)(((rb * 16 + lg * 4) * H * DV + col0 + ln) * 2), (e * H * DV + jb * 16) * 2, 0);
            }
#pragma unroll
            for (int i = 0; i < STW; ++i) {
                const int st = w + NW * i;
                if (st < NST) {
                    const int ct = st / NJT, jj = st % NJT;
                    f32x4 acc = zero4();
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const auto ff = M::ld32(sFT + (ct * 16 + ln) * LDC2 + s * 32 + lg * 8);
                        const auto fz = M::ld32(sZT + (jj * 16 + ln) * LDC2 + s * 32 + lg * 8);
                        acc = M::k32(ff, fz, acc);
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
        uint32_t any = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) any |= sBad[i];
        if (any) {
            WalkArgs wa{};
            wa.q = p.q; wa.k = p.k; wa.v = p.v; wa.alpha = p.alpha;
            wa.erase = gp.erase; wa.write = gp.write;
            wa.s0 = p.s0; wa.o = p.o; wa.sT = p.sT; wa.ckpt = nullptr;
            wa.H = H; wa.dv = DV; wa.gate = p.alpha ? 0 : 2; wa.fuse = 0; wa.scale = p.scale;
            __threadfence();  // this item's stores so far land before the walk's
            __syncthreads();
            token_walk<bf16_t, DK, DVT, NTH, true>(wa, seq, h, t0, len, col0,
                                                      reinterpret_cast<float*>(smem));
            return;
        }
    }

    if (p.sT) {
#pragma unroll
        for (int i = 0; i < STW; ++i) {
            const int st = w + NW * i;
            if (st < NST) {
                const int ct = st / NJT, jj = st % NJT;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    p.sT[sbase + (size_t)(ct * 16 + lg * 4 + e) * DV + col0 + jj * 16 + ln] = S[i][e];
            }
        }
    }
}

template <int DK, int DVT, int NW = 4>
hipError_t launch_g2(const G2Params& gp, hipStream_t stream) {
    using Lay = G2Layout<DK, DVT>;
    const int groups = (gp.base.units + 7) / 8;
    const long grid = 8L * gp.base.njt_all * groups;
    static const hipError_t attr = hipFuncSetAttribute(
        (const void*)gdn2_chunk_kernel<DK, DVT, NW>, hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gdn2_chunk_kernel<DK, DVT, NW>), dim3((unsigned)grid), dim3(NW * 64),
                       Lay::bytes, stream, gp);
    return hipGetLastError();
}

}  // namespace

// Value-column tile: the widest that still gives every compute unit a
// workgroup (at most 32 at dk = 128, where wider slices do not fit in LDS).
int plan_gdn2_dvt(int units, int dk, int dv) {
    const int widest = dk == 128 ? 32 : 64;
    for (int dvt = widest; dvt >= 16; dvt /= 2)
        if (dvt <= dv && (long)units * (dv / dvt) >= 256) return dvt;
    return 16;
}

hipError_t launch_gdn2_chunk_fwd(const Gdn2ChunkArgs& a, hipStream_t stream) {
    const int nseq = a.cu_seqlens ? a.num_seqs : a.B;
    const int units = nseq * a.H;
    if (units == 0) return hipSuccess;
    const int* order = nullptr;
    if (a.cu_seqlens && a.order) {
        hipError_t e = launch_order_sequences(a.cu_seqlens, a.num_seqs, a.order, stream);
        if (e != hipSuccess) return e;
        order = a.order;
    }
    int dvt = a.dvt > 0 ? a.dvt : plan_gdn2_dvt(units, a.dk, a.dv);
    if (dvt > a.dv) dvt = a.dv;
    if (a.dk == 128 && dvt > 32) dvt = 32;
    G2Params gp;
    KParams& p = gp.base;
    p.q = a.q; p.k = a.k; p.v = a.v; p.alpha = a.alpha; p.beta = nullptr; p.s0 = a.s0;
    p.o = a.o; p.sT = a.sT; p.cu_seqlens = a.cu_seqlens; p.order = order;
    p.B = a.B; p.T = a.T; p.H = a.H; p.dv = a.dv;
    p.units = units;
    p.njt_all = a.dv / dvt;
    p.gate = 0;
    p.fuse = 0;
    p.scale = a.scale;
    gp.erase = a.erase;
    gp.write = a.write;
    if (a.dk == 128) {
        // eight waves where each wave still gets a whole channel and value tile
        return dvt == 16 ? launch_g2<128, 16>(gp, stream) : launch_g2<128, 32, 8>(gp, stream);
    }
    switch (dvt) {
        case 16: return launch_g2<64, 16>(gp, stream);
        case 32: return launch_g2<64, 32>(gp, stream);
        default: return launch_g2<64, 64>(gp, stream);
    }
}

}  // namespace kda
