// chunk_fwd_bf16.hip -- the chunk-wise KDA forward for bf16 q/k/v on gfx950,
// organised as a pipeline of specialised waves inside each workgroup.
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
// Roles.  A workgroup owns one (unit, DVT value columns); its waves keep
// one role for the whole kernel:
//   consumers (waves 0..NJT-1): DVT/NJT columns of the fp32 state each, in
//     registers; they run the serial chain of chunk c (X, the solve, O, the
//     next state);
//   producers (4 waves, dk/4 key channels each): decays and the operands
//     Kr, Qr, Kc, Kc^T of chunk c+1, the q, k, alpha prefetch of chunk c+3,
//     and Gram blocks of chunk c+1;
//   helper: the inverses D_a and Pn of chunk c, beta and V^T of chunk c+1
//     (loaded a chunk earlier), and Gram blocks;
//   prefetch wave (last): touches the q, k, alpha and V lines of chunk c+3
//     so that the loads above find them in L2.
// In each segment the waves on its longest path (producers in segment 1,
// consumers in segment 2) take raised issue priority over the waves they
// share a SIMD with.
// Two workgroup barriers per chunk:
//   segment 1: consumers - O of chunk c-1; X and Qr (Pm*S0) of chunk c
//              producers - Kc^T(c); operands of chunk c+1; loads of chunk c+3
//              helper    - Pn(c); beta, V^T(c+1); loads of chunk c+2; D_a(c)
//   segment 2: consumers - solve, next state (O of chunk c follows in
//              segment 1 of chunk c+1, where the consumers have slack)
//              producers, helper - Gram blocks of chunk c+1
// What a segment writes and another segment of the same chunk reads is
// single-buffered; what is written one chunk ahead is double-buffered by
// chunk parity.
//
// Global memory is reached through buffer descriptors rebased per chunk whose
// range ends with the sequence's last row in the chunk: rows past the end of
// a sequence lie outside it, so their loads return zero and their stores are
// dropped.
#include "chunk_walk.h"

namespace kda {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

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
// Element offset of (row, channel) in a [64][LDK] token tile (LDK = dk + 8,
// so rows are 16 bytes longer than the data).  Bank behaviour of gfx950's LDS,
// measured with SQ_LDS_BANK_CONFLICT on probe kernels: a 16-byte read is served
// 16 lanes at a time over 64 four-byte banks, lanes 0-7 together with 16-23
// (and 8-15 with 24-31, ...); a 16-byte write, 16 consecutive lanes at a time.
// A matrix-core fragment read takes 8 rows x 2 column chunks per pass, a
// producer store 4 rows 4 apart x 4 chunks.  With dk = 128 (272-byte rows, 17
// chunks of 16 bytes) the data chunk c of row r is placed at chunk
// (c + 7 (r mod 2)) mod 16: row r then starts (in 16-byte bank groups) at
// r + 7 (r mod 2) = the even values 0..14 over any 8 consecutive rows, so
// both passes touch 16 distinct bank groups, where the plain layout gives every
// fragment read a 2-way conflict.  The rotation's reads need per-lane chunk
// offsets (formed once per wave where registers allow, ROT); otherwise (dk =
// 64, or an instance with no registers to spare) the 16-byte chunks of a row
// are XOR-swizzled by (row / 16) mod 4, which keeps the producers' stores
// apart and leaves the reads 2-way.
template <int LDK, bool ROT>
__device__ __forceinline__ int tok_off(int row, int ch) {
    if constexpr (ROT)
        return row * LDK + ((((ch >> 3) + 7 * (row & 1)) & 15) << 3) + (ch & 7);
    else
        return row * LDK + ((((ch >> 3) ^ (row >> 4)) & 3) | ((ch >> 3) & ~3)) * 8 + (ch & 7);
}
// Kc^T is kept with its rows (key channels) and columns (tokens) permuted
// inside groups of 32 so that matrix-core operands can be taken straight from
// accumulator registers.  A 16x16 accumulator tile gives lane (n, g) four
// consecutive indices 4g..4g+3 of its tile; two tiles t, t+1 together give the
// lane eight indices of one 32-group, which a 32-deep step consumes as the
// lane's run 8g..8g+7.  A contraction does not depend on how its index is
// ordered as long as both operands use one order, so:
//  - state tile ct, lane group g, element e holds key channel
//    32 (ct/2) + 8g + 4 (ct%2) + e; paired tiles then supply channels
//    32s + 8g + 0..7 in natural order, matching Kr and Qr;
//  - Kc^T row r holds the channel that the update's tile r/16 puts at row r%16;
//  - solve blocks 2s and 2s+1 supply tokens 32s + 4g + 0..3 and
//    32s + 16 + 4g + 0..3 as the run 8g..8g+7, so Kc^T column 32s + 8g + 4h + e
//    holds token 32s + 16h + 4g + e.
__device__ __forceinline__ int kct_row(int c) {  // Kc^T row of key channel c
    return ((c >> 5) * 2 + ((c >> 2) & 1)) * 16 + ((c >> 3) & 3) * 4 + (c & 3);
}
__device__ __forceinline__ int kct_col(int t) {  // Kc^T column of token t
    return (t & ~31) + ((t >> 2) & 3) * 8 + ((t >> 4) & 1) * 4 + (t & 3);
}
__device__ __forceinline__ int state_ch(int ct, int g, int e) {  // channel of S[ct][e] in lane group g
    return (ct >> 1) * 32 + g * 8 + (ct & 1) * 4 + e;
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
// Batched cross-lane steps over the N = 4 or 8 per-channel registers of a
// lane, one asm block each.  A DPP read needs two wait states after a VALU
// write of its source: one s_nop covers the first two registers of a block,
// and each later register was written at least N instructions earlier.
#define KDA_ARGS8(x) "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7])
#define KDA_ARGS4(x) "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])
#define KDA_SEQ8(OP) OP(0) OP(1) OP(2) OP(3) OP(4) OP(5) OP(6) OP(7)
#define KDA_SEQ4(OP) OP(0) OP(1) OP(2) OP(3)
#define KDA_SEQ1(OP) OP(0)
// x[i] *= x[i] of lane l - 4 (row_shr) or l - 4 mod 16 (row_ror) inside the
// lane's 16-lane row; with row_shr the first lanes of a row, which have no
// source, keep x[i]
#define KDA_MUL_DPP(NAME)                                                                       \
    __device__ __forceinline__ void NAME(float (&x)[8]) {                                       \
        asm volatile("s_nop 1\n\t" KDA_SEQ8(KDA_MUL_DPP_I_##NAME) : KDA_ARGS8(x));              \
    }                                                                                           \
    __device__ __forceinline__ void NAME(float (&x)[4]) {                                       \
        asm volatile("s_nop 1\n\t" KDA_SEQ4(KDA_MUL_DPP_I_##NAME) : KDA_ARGS4(x));              \
    }                                                                                           \
    __device__ __forceinline__ void NAME(float (&x)[1]) {                                       \
        asm volatile("s_nop 1\n\t" KDA_SEQ1(KDA_MUL_DPP_I_##NAME) : "+v"(x[0]));                \
    }
#define KDA_MUL_DPP_I_mul_row_shr4(i) "v_mul_f32_dpp %" #i ", %" #i ", %" #i " row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
#define KDA_MUL_DPP_I_mul_row_shr8(i) "v_mul_f32_dpp %" #i ", %" #i ", %" #i " row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
#define KDA_MUL_DPP_I_mul_row_ror8(i) "v_mul_f32_dpp %" #i ", %" #i ", %" #i " row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
KDA_MUL_DPP(mul_row_shr4)
KDA_MUL_DPP(mul_row_shr8)
KDA_MUL_DPP(mul_row_ror8)
// z[i] = x[i] * (x[i] of lane l - 4 mod 16 inside the row), into fresh registers
__device__ __forceinline__ void ror4_mul_into(float (&z)[8], const float (&x)[8]) {
    asm volatile("s_nop 1\n\t"
                 "v_mul_f32_dpp %0, %8, %8 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %1, %9, %9 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %2, %10, %10 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %3, %11, %11 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %4, %12, %12 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %5, %13, %13 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %6, %14, %14 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %7, %15, %15 row_ror:4 row_mask:0xf bank_mask:0xf"
                 : "=&v"(z[0]), "=&v"(z[1]), "=&v"(z[2]), "=&v"(z[3]), "=&v"(z[4]), "=&v"(z[5]), "=&v"(z[6]), "=&v"(z[7])
                 : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
}
__device__ __forceinline__ void ror4_mul_into(float (&z)[4], const float (&x)[4]) {
    asm volatile("s_nop 1\n\t"
                 "v_mul_f32_dpp %0, %4, %4 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %1, %5, %5 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %2, %6, %6 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %3, %7, %7 row_ror:4 row_mask:0xf bank_mask:0xf"
                 : "=&v"(z[0]), "=&v"(z[1]), "=&v"(z[2]), "=&v"(z[3])
                 : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
}
__device__ __forceinline__ void ror4_mul_into(float (&z)[1], const float (&x)[1]) {
    asm volatile("s_nop 1\n\t"
                 "v_mul_f32_dpp %0, %1, %1 row_ror:4 row_mask:0xf bank_mask:0xf"
                 : "=&v"(z[0])
                 : "v"(x[0]));
}
// f[i] *= w[i] of lane l - 4 inside the row; the first four lanes of a row
// keep f[i]
__device__ __forceinline__ void mul_shr4_from(float (&f)[8], const float (&w)[8]) {
    asm volatile("s_nop 1\n\t"
                 "v_mul_f32_dpp %0, %8, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %1, %9, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %2, %10, %2 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %3, %11, %3 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %4, %12, %4 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %5, %13, %5 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %6, %14, %6 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %7, %15, %7 row_shr:4 row_mask:0xf bank_mask:0xf"
                 : KDA_ARGS8(f)
                 : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]));
}
__device__ __forceinline__ void mul_shr4_from(float (&f)[4], const float (&w)[4]) {
    asm volatile("s_nop 1\n\t"
                 "v_mul_f32_dpp %0, %4, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %1, %5, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %2, %6, %2 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
                 "v_mul_f32_dpp %3, %7, %3 row_shr:4 row_mask:0xf bank_mask:0xf"
                 : KDA_ARGS4(f)
                 : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]));
}
__device__ __forceinline__ void mul_shr4_from(float (&f)[1], const float (&w)[1]) {
    asm volatile("s_nop 1\n\t"
                 "v_mul_f32_dpp %0, %1, %0 row_shr:4 row_mask:0xf bank_mask:0xf"
                 : "+v"(f[0])
                 : "v"(w[0]));
}
// exchange between 16-lane rows: (a, b) -> ([a0 b0 a2 b2], [a1 b1 a3 b3]) by
// rows, for each pair (a[i], b[i]); the trailing s_nop keeps the results two
// wait states away from a following DPP read
__device__ __forceinline__ void swap_rows16(float (&a)[8], float (&b)[8]) {
    asm volatile("s_nop 1\n\t"
                 "v_permlane16_swap_b32 %0, %8\n\t"
                 "v_permlane16_swap_b32 %1, %9\n\t"
                 "v_permlane16_swap_b32 %2, %10\n\t"
                 "v_permlane16_swap_b32 %3, %11\n\t"
                 "v_permlane16_swap_b32 %4, %12\n\t"
                 "v_permlane16_swap_b32 %5, %13\n\t"
                 "v_permlane16_swap_b32 %6, %14\n\t"
                 "v_permlane16_swap_b32 %7, %15\n\t"
                 "s_nop 1"
                 : KDA_ARGS8(a), KDA_ARGS8(b));
}
__device__ __forceinline__ void swap_rows16(float (&a)[4], float (&b)[4]) {
    asm volatile("s_nop 1\n\t"
                 "v_permlane16_swap_b32 %0, %4\n\t"
                 "v_permlane16_swap_b32 %1, %5\n\t"
                 "v_permlane16_swap_b32 %2, %6\n\t"
                 "v_permlane16_swap_b32 %3, %7\n\t"
                 "s_nop 1"
                 : KDA_ARGS4(a), KDA_ARGS4(b));
}
__device__ __forceinline__ void swap_rows16(float (&a)[1], float (&b)[1]) {
    asm volatile("s_nop 1\n\t"
                 "v_permlane16_swap_b32 %0, %1\n\t"
                 "s_nop 1"
                 : "+v"(a[0]), "+v"(b[0]));
}
#undef KDA_MUL_DPP
#undef KDA_MUL_DPP_I_mul_row_shr4
#undef KDA_MUL_DPP_I_mul_row_shr8
#undef KDA_MUL_DPP_I_mul_row_ror8
#undef KDA_SEQ8
#undef KDA_SEQ4
#undef KDA_SEQ1
#undef KDA_ARGS8
#undef KDA_ARGS4
// y in the 16-lane rows selected by ROWS (bit r = lanes 16r..16r+15), x elsewhere
template <int ROWS>
__device__ __forceinline__ float rows_sel(float x, float y) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(y), 0xE4, ROWS, 0xf, false));
}

template <int DK, int DVT, bool QN = false>
struct Lay6 {
    static constexpr int NJT = DVT >= 32 ? 2 : 1;  // consumer waves
    static constexpr int NT = DVT / 16 / NJT;      // 16-column state tiles per consumer
    static constexpr int NP = 4;               // producer waves
    static constexpr int CPL = DK / 16;        // key channels per producer lane
    static constexpr int NW = NJT + NP + 2;    // + the helper and the prefetch wave
    static constexpr int NTH = 64 * NW;
    static constexpr int RPV = DVT / 8;        // V rows per helper lane (8 columns each)
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
    static constexpr size_t bVT = bBeta + CH * 4;               // bf16 V^T [DVT][LDV]
    static constexpr size_t szBuf = (bVT + (size_t)DVT * LDV * 2 + 15) / 16 * 16;
    // single copies
    static constexpr size_t oKcT = 2 * szBuf;                   // [DK][LDC]
    static constexpr size_t oKc = oKcT + (size_t)DK * LDC * 2;  // [64][LDK]
    static constexpr size_t oLd = oKc + szTok;                  // fp32 [4][16 rows][LDL]
    static constexpr size_t oD = oLd + (size_t)4 * 16 * LDL * 4;  // D_a, 4 blocks row-major
    // with in-kernel q/k normalisation: fp32 partial sums of squares
    // [parity][q, k][64 rows][4 producers]
    static constexpr size_t oPart = oD + (size_t)4 * BLK * 2;
    // u32 [4]: a producer's chunks left the chunk form's range
    static constexpr size_t oBad = oPart + (QN ? (size_t)2 * 2 * CH * 4 * 4 : 0);
    static constexpr size_t bytes = oBad + 16;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// GATE: 0 = alpha per key channel (KDA), 1 = one alpha per token and head
// (Gated DeltaNet), 2 = no gate (DeltaNet, alpha = 1).
// FE: in-kernel input preparation, FUSE_GATE_LOGITS (bf16 logits z in place
// of alpha, alpha = sigmoid(z)) and FUSE_QK_L2NORM (q, k normalised per
// token); beta logits (FUSE_BETA_LOGITS) are a run-time flag.
// CKPT: the instance for the backward, which stores the state at every chunk
// start (p.ckpt) and may form no output (p.o NULL); kept apart so that the
// forward instances carry none of its code.
template <int DK, int DVT, int GATE, int FE, bool CKPT = false>
__global__ __launch_bounds__((Lay6<DK, DVT>::NTH), 1) void chunk_fwd_bf16_kernel(KParams p) {
    constexpr bool GL = (FE & FUSE_GATE_LOGITS) != 0, QN = (FE & FUSE_QK_L2NORM) != 0;
    static_assert(!(GL && GATE == 2), "gate logits need a gate");
    using L = Lay6<DK, DVT, QN>;
    using Mf = Mma<bf16_t>;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDB = L::LDB, LDL = L::LDL, BLK = L::BLK;
    constexpr int NJT = L::NJT, NT = L::NT, NP = L::NP, CPL = L::CPL, RPV = L::RPV;
    constexpr int NCT = DK / 16;          // 16-row tiles of a state slice

    extern __shared__ __align__(16) unsigned char smem[];
    auto buf = [&](int par, size_t off) { return smem + par * L::szBuf + off; };
    bf16_t* sKcT = reinterpret_cast<bf16_t*>(smem + L::oKcT);
    bf16_t* sKc = reinterpret_cast<bf16_t*>(smem + L::oKc);
    float* sLd = reinterpret_cast<float*>(smem + L::oLd);
    bf16_t* sD = reinterpret_cast<bf16_t*>(smem + L::oD);
    float* sPart = reinterpret_cast<float*>(smem + L::oPart);
    uint32_t* sBad = reinterpret_cast<uint32_t*>(smem + L::oBad);
    static_assert(WalkShape<DVT, L::NTH, false>::lds_bytes <= L::oBad, "walk LDS");

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
    // This lane's 16-byte chunk of row block rowblk at k-step s of a
    // matrix-fragment read of a token tile.  With the rotated layout the chunk
    // offsets within a row depend on the lane only (the row's parity is the
    // lane's), so they are formed once per wave and the reads need no per-step
    // address arithmetic; instances with in-kernel q/k normalisation have no
    // registers to spare for them and keep the XOR layout.
    constexpr bool ROT = DK == 128 && !QN;
    int fco[DK / 32];
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) fco[s] = ROT ? tok_off<LDK, ROT>(ln, s * 32 + lg * 8) - ln * LDK : 0;
    // (lane_n, lane_g: the caller's lane row and column group, used by the XOR
    // layout's address)
    auto frag_at = [&](const bf16_t* tile, int rowblk, int s, int lane_n, int lane_g) {
        if constexpr (ROT)
            return tile + (rowblk * 16 + ln) * LDK + fco[s];
        else
            return tile + tok_off<LDK, ROT>(rowblk * 16 + lane_n, s * 32 + lane_g * 8);
    };

    // byte strides of one token row
    const uint32_t rsq = (uint32_t)H * DK * 2, rsa = (uint32_t)H * DK * (GL ? 2 : 4);
    const uint32_t rsb = (uint32_t)H * 4, rsv = (uint32_t)H * DV * 2;
    // The transition part of a time segment (p.ident) reads no values: its
    // value descriptors get an empty range, so every load of v returns zero.
    const uint32_t vlim = p.ident ? 0u : ~0u;

    const bf16_t* __restrict__ gq = static_cast<const bf16_t*>(p.q);
    const bf16_t* __restrict__ gk = static_cast<const bf16_t*>(p.k);
    const bf16_t* __restrict__ gv = static_cast<const bf16_t*>(p.v);
    const float* __restrict__ ga = static_cast<const float*>(p.alpha);
    const bf16_t* __restrict__ gg = static_cast<const bf16_t*>(p.alpha);  // gate logits
    const float* __restrict__ gb = p.beta;

    // Every role ends in finish(): one barrier, after which the producers'
    // flags tell whether a chunk of this work item left the chunk form's range
    // (half-chunk decay product below 2^-100 in some key channel).  If one did,
    // redo() recomputes the work item's outputs and final state exactly, token
    // by token, with every wave of the workgroup.
    auto finish = [&]() -> bool {
        __syncthreads();
        return (sBad[0] | sBad[1] | sBad[2] | sBad[3]) != 0;
    };
    auto redo = [&]() {
        WalkArgs wa{};
        wa.q = p.q; wa.k = p.k; wa.v = p.v; wa.alpha = p.alpha; wa.beta = p.beta;
        wa.s0 = p.s0; wa.o = p.o; wa.sT = p.sT; wa.ckpt = p.ckpt; wa.ident = p.ident;
        wa.H = H; wa.dv = DV; wa.gate = GATE; wa.fuse = p.fuse; wa.scale = p.scale;
        __threadfence();  // this item's stores so far land before the walk's
        __syncthreads();
        token_walk<bf16_t, DK, DVT, L::NTH, false>(wa, wi.seq, h, t0, len, jt * DVT,
                                                   reinterpret_cast<float*>(smem));
    };

    // ---------------------------------------------------------- Gram blocks
    // Blocks (a, b), b <= a, of chunk ch: lane holds A[16a + ln][16b + 4lg + e]
    // and M likewise.  Diagonal blocks go to sLd (fp32, strictly lower part of
    // L_aa, row-major) and M; the others to -L_ab and M.  A worker takes
    // one or two blocks of one block row a, so the Kr and Qr fragments of the
    // row are read from LDS once for both.
    auto gram_out = [&](int par, int a, int b, f32x4 cA, f32x4 cM, float br, int ln, int lg) __attribute__((always_inline)) {
        bf16_t* m_b = reinterpret_cast<bf16_t*>(buf(par, L::bM));
        const int jn = a * (a + 1) / 2 + b;
        if (a == b) {
            f32x4 ld;
#pragma unroll
            for (int e = 0; e < 4; ++e) ld[e] = (lg * 4 + e < ln) ? br * cA[e] : 0.f;
            *reinterpret_cast<f32x4*>(sLd + (a * 16 + ln) * LDL + lg * 4) = ld;
            f32x4 mm;
#pragma unroll
            for (int e = 0; e < 4; ++e) mm[e] = (lg * 4 + e <= ln) ? cM[e] : 0.f;
            Mf::st4(m_b + jn * BLK + ln * LDB + lg * 4, mm);
        } else {
            f32x4 lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) lo[e] = -br * cA[e];
            Mf::st4(reinterpret_cast<bf16_t*>(buf(par, L::bLo)) + (a * (a - 1) / 2 + b) * BLK + ln * LDB + lg * 4, lo);
            Mf::st4(m_b + jn * BLK + ln * LDB + lg * 4, cM);
        }
    };
    auto gram_row = [&](int ch, int a, int b0, int nb) __attribute__((always_inline)) {  // blocks (a, b0 .. b0 + nb - 1)
        const int lx = (int)opaque((uint32_t)l);
        const int ln = lx & 15, lg = lx >> 4;
        const int par = ch & 1;
        const bf16_t* kr_b = reinterpret_cast<const bf16_t*>(buf(par, L::bKr));
        const bf16_t* qr_b = reinterpret_cast<const bf16_t*>(buf(par, L::bQr));
        f32x4 cA[2] = {zero4(), zero4()}, cM[2] = {zero4(), zero4()};
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            const auto fk = Mf::ld32(frag_at(kr_b, a, s, ln, lg));
            const auto fq = Mf::ld32(frag_at(qr_b, a, s, ln, lg));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (j < nb) {
                    const auto fa = Mf::ld32(frag_at(sKc, b0 + j, s, ln, lg));
                    cA[j] = Mf::k32(fa, fk, cA[j]);
                    cM[j] = Mf::k32(fa, fq, cM[j]);
                }
            }
        }
        const float br = reinterpret_cast<const float*>(buf(par, L::bBeta))[a * 16 + ln];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (j < nb) gram_out(par, a, b0 + j, cA[j], cM[j], br, ln, lg);
    };
    // worker k of the NP + 1 Gram workers (producers, then the helper):
    // rows 3 (two workers), 2 and 1 take two blocks each; the last worker
    // takes the diagonal blocks (2, 2) and (0, 0)
    auto gram_share = [&](int ch, int k) __attribute__((always_inline)) {
        static_assert(NP == 4, "five Gram workers");
        if (k == 0) gram_row(ch, 3, 0, 2);
        else if (k == 1) gram_row(ch, 3, 2, 2);
        else if (k == 2) gram_row(ch, 2, 0, 2);
        else if (k == 3) gram_row(ch, 1, 0, 2);
        else { gram_row(ch, 2, 2, 1); gram_row(ch, 0, 0, 1); }
    };

    if (w >= NJT && w < NJT + NP) {
        // ========================================================= producers
        // Lane (cq = l%4, rg = l/4) of producer pw owns key channels
        // pc0..pc0+CPL-1 and rows 4rg..4rg+3.  The four lanes of a quad read
        // one token's channels of this producer, so each load instruction
        // touches one 64-byte run per quad (one cache access, where lanes of
        // one channel group spread over rows would cost one access per lane);
        // 16-lane row r then holds tokens 16r..16r+15.
        const int pw = w - NJT;
        // decays per lane and row: one per channel, or one for the token
        constexpr int NA = GATE == 0 ? CPL : 1;
        // 32-bit words of raw alpha per lane and row (bf16 logits come in pairs)
        constexpr int NAW = GATE == 0 ? (GL ? CPL / 2 : CPL) : 1;
        // bytes per token of a per-head alpha
        const uint32_t rsh = (uint32_t)H * (GL ? 2 : 4);
        // registers carried across chunks: two sets of raw q, k, alpha rows
        // (chunks of even and odd index, loaded three chunks ahead) and the
        // Kc^T pairs of the chunk whose operands were built last
        struct Raw { uint32_t q[2 * CPL], k[2 * CPL], a[4 * NAW]; };
        Raw R0, R1;
        uint32_t RT[2 * CPL];
#pragma unroll
        for (int i = 0; i < 2 * CPL; ++i) { R0.q[i] = R0.k[i] = R1.q[i] = R1.k[i] = 0u; RT[i] = 0u; }
        bool pbad = false;  // a chunk's half-chunk decay product left the range
#pragma unroll
        for (int i = 0; i < 4 * NAW; ++i) R0.a[i] = R1.a[i] = 0u;

        // descriptors and lane offsets of the raw q, k, alpha rows of chunk ch
        struct Src { Rsrc rq, rk, ra; uint32_t qo, ao; };
        auto p_src = [&](int ch) {
            const int lx = (int)opaque((uint32_t)l);
            const int pc0 = pw * (DK / 4) + (lx & 3) * CPL, pr0 = (lx >> 2) * 4;
            const size_t e0 = ((size_t)(t0 + (long)ch * CH) * H + h) * DK;
            // rows of this chunk inside the sequence (0 past the last chunk: the
            // loads then fall outside the range, read nothing and return zero;
            // issuing them anyway keeps the count of loads in flight the same
            // on every path, so the waits for them stay exact)
            const int nr = __builtin_amdgcn_readfirstlane(max(0, min(len - ch * CH, CH)));
            Src sr;
            sr.rq = make_rsrc(gq + e0, (uint32_t)nr * rsq);
            sr.rk = make_rsrc(gk + e0, (uint32_t)nr * rsq);
            sr.qo = (uint32_t)pr0 * rsq + (uint32_t)pc0 * 2;
            if constexpr (GATE == 0) {
                sr.ra = make_rsrc(GL ? (const void*)(gg + e0) : (const void*)(ga + e0), (uint32_t)nr * rsa);
                sr.ao = (uint32_t)pr0 * rsa + (uint32_t)pc0 * (GL ? 2 : 4);
            } else {  // alpha [token][head]; unused without a gate
                const void* hb = GL ? (const void*)(gg + e0 / DK) : (const void*)(ga + e0 / DK);
                sr.ra = make_rsrc(GATE == 1 ? hb : p.alpha, GATE == 1 ? (uint32_t)nr * rsh : 0u);
                sr.ao = (uint32_t)pr0 * rsh;
            }
            return sr;
        };
        auto ld_qk = [&](const Src& sr, Raw& R, int rr) {  // q and k of the lane's row rr
            if constexpr (CPL == 8) {
                const u32x4 q4 = __builtin_amdgcn_raw_buffer_load_b128(sr.rq, sr.qo + rr * rsq, 0, 0);
                const u32x4 k4 = __builtin_amdgcn_raw_buffer_load_b128(sr.rk, sr.qo + rr * rsq, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) { R.q[4 * rr + i] = q4[i]; R.k[4 * rr + i] = k4[i]; }
            } else {
                const u32x2 q2 = __builtin_amdgcn_raw_buffer_load_b64(sr.rq, sr.qo + rr * rsq, 0, 0);
                const u32x2 k2 = __builtin_amdgcn_raw_buffer_load_b64(sr.rk, sr.qo + rr * rsq, 0, 0);
                R.q[2 * rr] = q2[0]; R.q[2 * rr + 1] = q2[1];
                R.k[2 * rr] = k2[0]; R.k[2 * rr + 1] = k2[1];
            }
        };
        auto ld_a = [&](const Src& sr, Raw& R, int rr) {  // alpha of the lane's row rr
            if constexpr (GATE == 0 && !GL) {
#pragma unroll
                for (int j = 0; j < CPL / 4; ++j) {
                    const u32x4 a4 = __builtin_amdgcn_raw_buffer_load_b128(sr.ra, sr.ao + rr * rsa + 16 * j, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) R.a[CPL * rr + 4 * j + i] = a4[i];
                }
            } else if constexpr (GATE == 0 && CPL == 8) {  // 8 bf16 logits
                const u32x4 a4 = __builtin_amdgcn_raw_buffer_load_b128(sr.ra, sr.ao + rr * rsa, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) R.a[4 * rr + i] = a4[i];
            } else if constexpr (GATE == 0) {  // 4 bf16 logits
                const u32x2 a2 = __builtin_amdgcn_raw_buffer_load_b64(sr.ra, sr.ao + rr * rsa, 0, 0);
                R.a[2 * rr] = a2[0]; R.a[2 * rr + 1] = a2[1];
            } else if constexpr (GATE == 1 && !GL) {
                R.a[rr] = __builtin_amdgcn_raw_buffer_load_b32(sr.ra, sr.ao + rr * rsh, 0, 0);
            } else if constexpr (GATE == 1) {  // one bf16 logit, in the low half
                R.a[rr] = __builtin_amdgcn_raw_buffer_load_b16(sr.ra, sr.ao + rr * rsh, 0, 0);
            }
        };
        auto p_load = [&](int ch, Raw& R) {  // raw q, k, alpha rows of chunk ch
            const Src sr = p_src(ch);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) { ld_qk(sr, R, rr); ld_a(sr, R, rr); }
        };
        // Partial sums of squares of the raw q and k rows of chunk ch held in R,
        // over this producer's channels, into sPart (parity ch & 1): a quad's
        // four lanes hold one token's channels of the producer, so two DPP
        // steps finish the producer's sum and the first lane stores it.
        auto p_norms = [&](const Raw& R, int ch) {
            const int lx = (int)opaque((uint32_t)l);
            const int pr0 = (lx >> 2) * 4;
            float ss[2][4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int i = 0; i < CPL / 2; ++i) {
                    const bf16x2v qw = __builtin_bit_cast(bf16x2v, R.q[(CPL / 2) * rr + i]);
                    const bf16x2v kw = __builtin_bit_cast(bf16x2v, R.k[(CPL / 2) * rr + i]);
                    sq = __builtin_amdgcn_fdot2_f32_bf16(qw, qw, sq, false);
                    sk = __builtin_amdgcn_fdot2_f32_bf16(kw, kw, sk, false);
                }
                ss[0][rr] = sq;
                ss[1][rr] = sk;
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    float x = ss[t][rr];
                    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));
                    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));
                    ss[t][rr] = x;
                }
            if ((lx & 3) == 0) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        sPart[(((ch & 1) * 2 + t) * CH + pr0 + rr) * 4 + pw] = ss[t][rr];
            }
        };
        auto p_write_kct = [&]() {
            const int lx = (int)opaque((uint32_t)l);
            const int pc0 = pw * (DK / 4) + (lx & 3) * CPL, pr0 = (lx >> 2) * 4;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                *reinterpret_cast<uint2*>(sKcT + kct_row(pc0 + c) * LDC + kct_col(pr0)) =
                    make_uint2(RT[2 * c], RT[2 * c + 1]);
        };
        // Decayed operands of chunk ch into parity buffer ch & 1 (Kc^T kept in
        // RT).  The raw rows of chunk chl are loaded into R as its rows of
        // chunk ch are used up, so the loads spread over the computation.
        auto p_operands = [&](int ch, Raw& R, int chl) {
            const Src sr = p_src(chl);
            uint32_t* RQ = R.q;
            uint32_t* RK = R.k;
            uint32_t* RA = R.a;
            auto ra_f = [&](int i) { return __uint_as_float(RA[i]); };
            const int lx = (int)opaque((uint32_t)l);
            const int rg = lx >> 2;
            const int pc0 = pw * (DK / 4) + (lx & 3) * CPL, pr0 = rg * 4;
            const int par = ch & 1;
            const int nval = len - ch * CH;
            bf16_t* kr_b = reinterpret_cast<bf16_t*>(buf(par, L::bKr));
            bf16_t* qr_b = reinterpret_cast<bf16_t*>(buf(par, L::bQr));
            // decays: f (P through row pr0 - 1, over Pm), g (Pm / P through row
            // pr0 + 3), the running products pr over the lane's rows, and u (Pm
            // in 16-lane row 0, Pn / Pm in row 3); index ai(c) for channel c
            auto ai = [](int c) { return GATE == 0 ? c : 0; };
            // The decays of the lane's rows: stored alpha, or from the stored
            // logits, formed once here (rows past the end decay by 1).  From
            // per-channel logits the scan below runs on 1 / alpha = 1 + e^-z,
            // which needs no reciprocal per element: every product it forms is
            // then the inverse of the one it stands for, so P_r / Pm and
            // Pm / P_r trade places and the vector entries are inverted.
            constexpr bool INV = GL && GATE == 0;
            float al[GL ? 4 : 1][GL ? NA : 1];
            if constexpr (GL) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                    for (int c = 0; c < NA; ++c) {
                        const uint32_t wd = RA[NAW * rr + c / 2];
                        const float z = (c & 1) ? hi_f(wd) : lo_f(wd);
                        if constexpr (INV)
                            al[rr][c] = (pr0 + rr < nval) ? 1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z) : 1.f;
                        else
                            al[rr][c] = (pr0 + rr < nval) ? sigmoid_f(z) : 1.f;
                    }
            }
            auto alv = [&](int rr, int c) {
                if constexpr (GL) return al[rr][c];
                else return ra_f(NA * rr + c);
            };
            // 1 / |k| and 1 / |q| of the lane's rows from the producers' partial sums
            float ik[4], iq[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                ik[rr] = iq[rr] = 1.f;
                if constexpr (QN) {
                    const float4 sq = ld4(sPart + (((ch & 1) * 2 + 0) * CH + pr0 + rr) * 4);
                    const float4 sk = ld4(sPart + (((ch & 1) * 2 + 1) * CH + pr0 + rr) * 4);
                    iq[rr] = inv_norm((sq.x + sq.y) + (sq.z + sq.w));
                    ik[rr] = inv_norm((sk.x + sk.y) + (sk.z + sk.w));
                }
            }
            float pr[4][NA], f[NA], g[NA], u[NA];
            if constexpr (GATE == 2) {
#pragma unroll
                for (int c = 0; c < NA; ++c) {
                    f[c] = g[c] = u[c] = 1.f;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) pr[rr][c] = 1.f;
                }
            } else {
                if (!GL && nval < CH) {  // alpha of rows past the end of the sequence is 1
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        if (pr0 + rr >= nval)
#pragma unroll
                            for (int c = 0; c < NA; ++c) RA[NA * rr + c] = __float_as_uint(1.f);
                }
                float inc[NA];
#pragma unroll
                for (int c = 0; c < NA; ++c) {
                    float run = alv(0, c);
                    pr[0][c] = run;
#pragma unroll
                    for (int rr = 1; rr < 4; ++rr) { run *= alv(rr, c); pr[rr][c] = run; }
                    inc[c] = run;
                }
                ld_a(sr, R, 0);  // alpha of row 0 is used up
                __builtin_amdgcn_sched_barrier(0);  // keep each batch of loads where it is issued
                // Products over the chunk's tokens, per channel.  w: over the
                // lane's 16-lane row through its last token (tokens 16r..pr0+3);
                // z: over the whole row (tokens 16r..16r+15), in every lane.
                float w[NA], z[NA];
#pragma unroll
                for (int c = 0; c < NA; ++c) w[c] = inc[c];
                mul_row_shr4(w);
                mul_row_shr8(w);
                ror4_mul_into(z, inc);
                mul_row_ror8(z);
                // With row totals z0..z3, Pm = z0 z1 and P_t / Pm = w_t F where F
                // is 1/(z0 z1), 1/z1, 1 and z2 in rows 0..3.  The row exchange
                // gives a = (z0, z0, z2, z2) and b = (z1, z1, z3, z3) by row; with
                // t = (z0, 1, 1, z2), u = t b is Pm in row 0 and Pn / Pm in row 3.
                float a[NA];
#pragma unroll
                for (int c = 0; c < NA; ++c) a[c] = z[c];
                swap_rows16(a, z);  // z now holds b
#pragma unroll
                for (int c = 0; c < NA; ++c) {
                    const float t = rows_sel<0x6>(a[c], 1.f);
                    u[c] = t * z[c];
                    f[c] = rows_sel<0xC>(fast_rcp(u[c]), t);  // F
                    g[c] = fast_rcp(w[c] * f[c]);            // Pm / P through row pr0 + 3
                }
                mul_shr4_from(f, w);  // P through row pr0 - 1, over Pm
                // range check on Pm (row 0) and Pn / Pm (row 3); the scan on
                // 1 / alpha holds their inverses, which overflow instead
                if ((lx >> 4) == 0 || (lx >> 4) == 3) {
#pragma unroll
                    for (int c = 0; c < NA; ++c)
                        pbad |= INV ? u[c] > 1.f / DECAY_FLOOR : u[c] < DECAY_FLOOR;
                }
            }
            // Pm from the first lanes of row 0, Pn / Pm from the first lanes of
            // row 3; the helper forms Pn from the two
            if (rg == 0 || rg == 12) {
                float* vec = reinterpret_cast<float*>(buf(par, L::bVec)) + (rg == 0 ? 0 : 2 * DK);
#pragma unroll
                for (int c = 0; c < CPL; c += 4) {
                    float4 v4 = make_float4(u[ai(c)], u[ai(c + 1)], u[ai(c + 2)], u[ai(c + 3)]);
                    if constexpr (INV)
                        v4 = make_float4(fast_rcp(v4.x), fast_rcp(v4.y), fast_rcp(v4.z), fast_rcp(v4.w));
                    *reinterpret_cast<float4*>(vec + pc0 + c) = v4;
                }
            }
            // rows from the last to the first: g_r = Pm / P_r = g_{r+1} * alpha_{r+1}
            uint32_t kcp[CPL / 2];  // Kc of row rr + 1 (the odd row of the current pair)
#pragma unroll
            for (int rr = 3; rr >= 0; --rr) {
                uint32_t kr[CPL / 2], qr[CPL / 2], kc[CPL / 2];
                if constexpr (GATE == 1) {
                    if (rr < 3) g[0] *= alv(rr + 1, 0);
                }
                const float rrow = pr[rr][0] * f[0];  // P_r / Pm of a token-wide decay
                // row multipliers with the norms folded in (the norms are 1 without QN)
                const float rrk = rrow * ik[rr], rrq = rrow * iq[rr], grk = g[0] * ik[rr];
#pragma unroll
                for (int i = 0; i < CPL / 2; ++i) {
                    const uint32_t kw = RK[(CPL / 2) * rr + i], qw = RQ[(CPL / 2) * rr + i];
                    const int c0 = 2 * i, c1 = 2 * i + 1;
                    if constexpr (GATE == 2 && !QN) {  // no decay: the stored values as they are
                        kr[i] = kw;
                        qr[i] = qw;
                        kc[i] = kw;
                    } else if constexpr (GATE == 2) {  // normalised, no decay
                        kr[i] = pack2(lo_f(kw) * ik[rr], hi_f(kw) * ik[rr]);
                        qr[i] = pack2(lo_f(qw) * iq[rr], hi_f(qw) * iq[rr]);
                        kc[i] = kr[i];
                    } else if constexpr (GATE == 0) {
                        if (rr < 3) {
                            g[c0] *= alv(rr + 1, c0);
                            g[c1] *= alv(rr + 1, c1);
                        }
                        const float p0 = pr[rr][c0] * f[c0], p1 = pr[rr][c1] * f[c1];
                        // P_r / Pm and Pm / P_r (swapped when the scan ran on 1 / alpha)
                        const float r0 = INV ? g[c0] : p0, r1 = INV ? g[c1] : p1;
                        const float h0 = INV ? p0 : g[c0], h1 = INV ? p1 : g[c1];
                        float k0 = lo_f(kw), k1 = hi_f(kw), q0 = lo_f(qw), q1 = hi_f(qw);
                        if constexpr (QN) {
                            k0 *= ik[rr]; k1 *= ik[rr];
                            q0 *= iq[rr]; q1 *= iq[rr];
                        }
                        kr[i] = pack2(k0 * r0, k1 * r1);
                        qr[i] = pack2(q0 * r0, q1 * r1);
                        kc[i] = pack2(k0 * h0, k1 * h1);
                    } else {  // one decay for the token
                        const float k0 = lo_f(kw), k1 = hi_f(kw);
                        kr[i] = pack2(k0 * rrk, k1 * rrk);
                        qr[i] = pack2(lo_f(qw) * rrq, hi_f(qw) * rrq);
                        kc[i] = pack2(k0 * grk, k1 * grk);
                    }
                    if (rr & 1) {
                        kcp[i] = kc[i];
                    } else {  // Kc^T pairs of channels c0, c1: rows (rr, rr + 1)
                        RT[2 * c0 + (rr >> 1)] = __builtin_amdgcn_perm(kcp[i], kc[i], 0x05040100u);
                        RT[2 * c1 + (rr >> 1)] = __builtin_amdgcn_perm(kcp[i], kc[i], 0x07060302u);
                    }
                }
                const int to = tok_off<LDK, ROT>(pr0 + rr, pc0);
                if constexpr (CPL == 8) {
                    *reinterpret_cast<uint4*>(kr_b + to) = make_uint4(kr[0], kr[1], kr[2], kr[3]);
                    *reinterpret_cast<uint4*>(qr_b + to) = make_uint4(qr[0], qr[1], qr[2], qr[3]);
                    *reinterpret_cast<uint4*>(sKc + to) = make_uint4(kc[0], kc[1], kc[2], kc[3]);
                } else {
                    *reinterpret_cast<uint2*>(kr_b + to) = make_uint2(kr[0], kr[1]);
                    *reinterpret_cast<uint2*>(qr_b + to) = make_uint2(qr[0], qr[1]);
                    *reinterpret_cast<uint2*>(sKc + to) = make_uint2(kc[0], kc[1]);
                }
                ld_qk(sr, R, rr);                 // q, k of row rr are used up
                if (rr < 3) ld_a(sr, R, rr + 1);  // and alpha of row rr + 1
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // Every producer step runs unconditionally.  Past the last chunk its
        // loads return zero and it writes zero operands into the parity buffer
        // nobody reads any more; in exchange no path skips a load or a use of
        // loaded registers, which keeps the waits for loads in flight exact.
        //   segment 1: Kc^T(c); operands of c+1 from its raw set, which
        //              meanwhile receives the rows of c+3
        //   segment 2: Gram blocks of c+1
        auto step = [&](int ch, Raw& R, const Raw& RO) {
            __builtin_amdgcn_s_setprio(2);
            p_write_kct();  // Kc^T of chunk ch (its Kc came with the operands one chunk ago)
            p_operands(ch + 1, R, ch + 3);
            if constexpr (QN) p_norms(RO, ch + 2);  // RO holds the rows of chunk ch + 2
            __syncthreads();
            __builtin_amdgcn_s_setprio(0);
            gram_share(ch + 1, pw);
            __syncthreads();
        };
        p_load(0, R0);
        p_load(1, R1);
        if constexpr (QN) {
            p_norms(R0, 0);
            p_norms(R1, 1);
            __syncthreads();
        }
        p_operands(0, R0, 2);
        __syncthreads();
        gram_share(0, pw);
        __syncthreads();
        // two chunks per trip so each raw set keeps fixed registers
        int ch = 0;
        for (; ch + 1 < nch; ch += 2) {
            step(ch, R1, R0);
            step(ch + 1, R0, R1);
        }
        if (ch < nch) step(ch, R1, R0);
        const uint64_t bad = __builtin_amdgcn_ballot_w64(pbad);
        if (l == 0) sBad[pw] = bad != 0;
        if (finish()) redo();
        return;
    }

    if (w == NJT + NP) {
        // ============================================================ helper
        // beta of a chunk (lane = row) and its V slice: lane (cg = l % (DVT/8),
        // rq = l / (DVT/8)) holds rows RPV*rq .. +RPV-1, slice columns
        // 8cg..8cg+7 (consecutive lanes read one row's columns, so the loads
        // coalesce)
        uint32_t HB = 0u, HV[4 * RPV];
#pragma unroll
        for (int i = 0; i < 4 * RPV; ++i) HV[i] = 0u;
        auto h_load = [&](int ch) {  // beta and V rows of chunk ch (zero past the end)
            const int lx = (int)opaque((uint32_t)l);
            const int rq = lx / (DVT / 8), cg = lx % (DVT / 8);
            const int nr = __builtin_amdgcn_readfirstlane(max(0, min(len - ch * CH, CH)));
            const size_t tok = (size_t)(t0 + (long)ch * CH) * H + h;
            const Rsrc rb = make_rsrc(gb + tok, (uint32_t)nr * rsb);
            HB = __builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)lx * rsb, 0, 0);
            const Rsrc rv = make_rsrc(gv + tok * DV + jt * DVT, ((uint32_t)nr * rsv) & vlim);
            const uint32_t vo = (uint32_t)(RPV * rq) * rsv + (uint32_t)cg * 16;
#pragma unroll
            for (int i = 0; i < RPV; ++i) {
                const u32x4 v4 = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + i * rsv, 0, 0);
                HV[4 * i] = v4[0]; HV[4 * i + 1] = v4[1]; HV[4 * i + 2] = v4[2]; HV[4 * i + 3] = v4[3];
            }
        };
        auto h_pn = [&](int ch) {  // Pn = Pm (Pn / Pm) of chunk ch, per key channel
            float* vec = reinterpret_cast<float*>(buf(ch & 1, L::bVec));
            const int lx = (int)opaque((uint32_t)l);
#pragma unroll
            for (int c = 0; c < DK / 64; ++c) {
                const int kc = lx + 64 * c;
                vec[DK + kc] = vec[kc] * vec[2 * DK + kc];
            }
        };
        auto h_write_beta = [&](int ch) {
            const int lx = (int)opaque((uint32_t)l);
            float bv = __uint_as_float(HB);
            // beta logits: sigmoid for the rows of the chunk; rows past the end keep 0
            if ((p.fuse & FUSE_BETA_LOGITS) && lx < len - ch * CH) bv = sigmoid_f(bv);
            reinterpret_cast<float*>(buf(ch & 1, L::bBeta))[lx] = bv;
        };
        // V^T: for each of the lane's 8 columns, its RPV rows as one run
        auto h_write_vt = [&](int ch) {
            const int lx = (int)opaque((uint32_t)l);
            const int rq = lx / (DVT / 8), cg = lx % (DVT / 8);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                bf16_t* dst = reinterpret_cast<bf16_t*>(buf(ch & 1, L::bVT)) + (cg * 8 + c) * L::LDV + RPV * rq;
                uint32_t wr[RPV / 2];  // rows 2i, 2i + 1 of column c
#pragma unroll
                for (int i = 0; i < RPV / 2; ++i)
                    wr[i] = __builtin_amdgcn_perm(HV[4 * (2 * i + 1) + c / 2], HV[4 * (2 * i) + c / 2], sel);
                // the V^T pitch keeps runs 8-byte aligned only
#pragma unroll
                for (int i = 0; i < RPV / 2; i += 2)
                    store_run<uint32_t, (RPV / 2 < 2 ? RPV / 2 : 2)>(reinterpret_cast<uint32_t*>(dst) + i, wr + i);
            }
        };
        // D_a = (I + L_aa)^{-1} of the chunk whose diagonal blocks are in sLd:
        // lane (block lg, row ln) forms row ln of D_a from D (I + L) = I,
        // right-looking from the last column: once x[k] = D[ln][k] is final,
        // x[k] L[k][j] leaves every x[j], j < k.  The 15 steps each read one
        // row of L_aa (the same for the 16 lanes of a block) and the row of
        // D goes out as two 16-byte stores.
        auto h_dsolve = [&]() {
            const int lx = (int)opaque((uint32_t)l);
            const int ln = lx & 15, lg = lx >> 4;
            float x[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) x[k] = (k == ln) ? 1.f : 0.f;
            const float* La = sLd + lg * 16 * LDL;
#pragma unroll
            for (int k = 15; k >= 1; --k) {
                float row[16];
#pragma unroll
                for (int q4 = 0; q4 < (k + 3) / 4; ++q4) {
                    const float4 v = ld4(La + k * LDL + q4 * 4);
                    row[q4 * 4] = v.x; row[q4 * 4 + 1] = v.y; row[q4 * 4 + 2] = v.z; row[q4 * 4 + 3] = v.w;
                }
#pragma unroll
                for (int j = 0; j < k; ++j) x[j] -= x[k] * row[j];
            }
            bf16_t* dr = sD + lg * BLK + ln * LDB;
            *reinterpret_cast<uint4*>(dr) = make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
            *reinterpret_cast<uint4*>(dr + 8) =
                make_uint4(pack2(x[8], x[9]), pack2(x[10], x[11]), pack2(x[12], x[13]), pack2(x[14], x[15]));
        };
        h_load(0);
        h_write_beta(0);
        h_write_vt(0);
        h_load(1);
        if constexpr (QN) __syncthreads();
        __syncthreads();
        gram_share(0, NP);
        __syncthreads();
        for (int ch = 0; ch < nch; ++ch) {
            // segment 1: Pn of chunk ch; beta and V^T of chunk ch + 1 into its
            // parity buffer, loads of chunk ch + 2, then D of chunk ch
            h_pn(ch);
            h_write_beta(ch + 1);
            h_write_vt(ch + 1);
            h_load(ch + 2);
            h_dsolve();
            __syncthreads();
            // segment 2
            gram_share(ch + 1, NP);
            __syncthreads();
        }
        if (finish()) redo();
        return;
    }

    if (w == NJT + NP + 1) {
        // ====================================================== prefetch wave
        // Pulls the q, k, alpha and V lines of chunk c + 3 into L2 at the start of
        // chunk c, so that the producers' loads of them (spread over the operand
        // build later in the same segment) and the helper's (chunk c + 1) find
        // them in L2 or in flight instead of waiting out HBM latency with some
        // 500 lines in flight per compute unit.  Value tile jt of a unit takes
        // rows jt*64/njt.. of the chunk, one line per lane and tensor; the
        // four tiles together touch every line once.  Three register sets
        // rotate, so a wait for a set's loads comes three chunks after them.
        uint32_t P0[4] = {0u, 0u, 0u, 0u}, P1[4] = {0u, 0u, 0u, 0u}, P2[4] = {0u, 0u, 0u, 0u};
        auto pf = [&](int ch, uint32_t (&r)[4]) {
            const int lx = (int)opaque((uint32_t)l);
            const int njt = p.njt_all;
            const int nr = __builtin_amdgcn_readfirstlane(max(0, min(len - ch * CH, CH)));
            const size_t tok = (size_t)(t0 + (long)ch * CH) * H + h;
            const uint32_t row = (uint32_t)(jt * (CH / njt) + lx / njt), sub = (uint32_t)(lx % njt);
            const Rsrc rq = make_rsrc(gq + tok * DK, (uint32_t)nr * rsq);
            const Rsrc rk = make_rsrc(gk + tok * DK, (uint32_t)nr * rsq);
            const Rsrc rv = make_rsrc(gv + tok * DV, ((uint32_t)nr * rsv) & vlim);
            r[0] = __builtin_amdgcn_raw_buffer_load_b32(rq, row * rsq + (sub & 1) * 128, 0, 0);
            r[1] = __builtin_amdgcn_raw_buffer_load_b32(rk, row * rsq + (sub & 1) * 128, 0, 0);
            if constexpr (GATE == 0) {  // 512-byte rows (256 with bf16 logits)
                const Rsrc ra = make_rsrc(GL ? (const void*)(gg + tok * DK) : (const void*)(ga + tok * DK),
                                          (uint32_t)nr * rsa);
                r[2] = __builtin_amdgcn_raw_buffer_load_b32(ra, row * rsa + (sub & (GL ? 1 : 3)) * 128, 0, 0);
            } else if constexpr (GATE == 1) {
                const uint32_t rsh = (uint32_t)H * (GL ? 2 : 4);
                const Rsrc ra = make_rsrc(GL ? (const void*)(gg + tok) : (const void*)(ga + tok), (uint32_t)nr * rsh);
                if constexpr (GL)  // bf16 logits: 2-byte elements
                    r[2] = __builtin_amdgcn_raw_buffer_load_b16(ra, row * rsh, 0, 0);
                else
                    r[2] = __builtin_amdgcn_raw_buffer_load_b32(ra, row * rsh, 0, 0);
            } else {
                r[2] = 0u;
            }
            r[3] = __builtin_amdgcn_raw_buffer_load_b32(rv, row * rsv + (sub & 1) * 128, 0, 0);
        };
        if constexpr (QN) __syncthreads();
        __syncthreads();
        __syncthreads();
        int ch = 0;
        for (; ch + 2 < nch; ch += 3) {
            pf(ch + 3, P0);
            __syncthreads();
            __syncthreads();
            pf(ch + 4, P1);
            __syncthreads();
            __syncthreads();
            pf(ch + 5, P2);
            __syncthreads();
            __syncthreads();
        }
        for (; ch < nch; ++ch) {
            __syncthreads();
            __syncthreads();
        }
        asm volatile("" :: "v"(P0[0]), "v"(P0[1]), "v"(P0[2]), "v"(P0[3]), "v"(P1[0]), "v"(P1[1]), "v"(P1[2]),
                     "v"(P1[3]), "v"(P2[0]), "v"(P2[1]), "v"(P2[2]), "v"(P2[3]));
        if (finish()) redo();
        return;
    }

    // ============================================================ consumers
    // The consumers carry the serial state chain.  In segment 2 it is the
    // longest path, so the SIMD arbiter is told to prefer them there over the
    // producers they share a SIMD with; in segment 1 they take the lowest
    // priority unless they hold two tiles.  Consumer cj holds NT 16-column tiles of the state;
    // with NT = 2 (DVT 64) the tiles share every fragment read and their
    // independent chains interleave.
    // The state, U and Pm*S stay in registers: the operand orders set out at
    // kct_row let each product take them as they are.
    const int cj = w;                                // consumer
    const int colw = jt * DVT + cj * 16 * NT;        // first value column of this wave
    const int col = colw + ln;                       // this lane's value column in tile 0
    bf16_t* __restrict__ go = static_cast<bf16_t*>(p.o);
    const size_t sbase = ((size_t)wi.seq * H + h) * DK * DV;

    f32x4 S[NT][NCT], Y[NT][4], OI[NT][4];  // state, beta-scaled X, (Qr (Pm S0))^T
    // this wave's columns of the state into a float32 [dk][dv] block
    // (lane offsets recomputed per call, so no per-element address stays live;
    // checkpoints are read back only by the reverse sweep, long after, so they
    // are stored non-temporally)
    auto store_state = [&](float* dst) {
        const int lx = (int)opaque((uint32_t)l);
        float* base = dst + (size_t)(lx >> 4) * 8 * DV + colw + (lx & 15);
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float* q = base + (size_t)state_ch(ct, 0, e) * DV + 16 * j;
                    if constexpr (CKPT) __builtin_nontemporal_store(S[j][ct][e], q);
                    else *q = S[j][ct][e];
                }
    };
    const size_t slot0 = (size_t)(t0 / CH + 2 * (long)wi.seq);
    auto ckpt_at = [&](int ch) { return p.ckpt + ((slot0 + ch) * H + h) * DK * DV; };
    Mf::F16 UP[NT][4];                      // U of the last solved chunk (B operand layout)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            S[j][ct] = zero4();
            if (p.ident) {  // the identity's columns (dv == dk)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[j][ct][e] = state_ch(ct, lg, e) == col + 16 * j ? 1.f : 0.f;
            } else if (p.s0) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[j][ct][e] = p.s0[sbase + (size_t)state_ch(ct, lg, e) * DV + col + 16 * j];
            }
        }
    // O_a = scale (OI_a + sum_{b<=a} M_ab U_b) of chunk ch, one 16-token block
    // of U per step; run in the consumers' first segment of chunk ch + 1 (M and
    // OI of chunk ch are still in place there) or after the last chunk.  The
    // products are taken with their operands swapped, which yields O_a^T: lane
    // (n, g) then holds value columns 4g..4g+3 of token n, one 8-byte store.
    auto c_out = [&](int ch) {
        if constexpr (CKPT) {
            if (!go) return;  // a call that only stores checkpoints
        }
        const int lx = (int)opaque((uint32_t)l);
        const int ln = lx & 15, lg = lx >> 4;
        const bf16_t* m_b = reinterpret_cast<const bf16_t*>(buf(ch & 1, L::bM));
        const Rsrc ro = make_rsrc(go + ((size_t)(t0 + (long)ch * CH) * H + h) * DV + colw,
                                  (uint32_t)min(len - ch * CH, CH) * rsv);
        const uint32_t ob = (uint32_t)ln * rsv + (uint32_t)lg * 8;  // token ln, column colw + 4lg
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4 co[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) co[j] = OI[j][a];
#pragma unroll
            for (int b = 0; b <= a; ++b) {
                const auto fm = Mf::ld16(m_b + (a * (a + 1) / 2 + b) * BLK + ln * LDB + lg * 4);
#pragma unroll
                for (int j = 0; j < NT; ++j) co[j] = Mf::k16(UP[j][b], fm, co[j]);
            }
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const u32x2 ow = {pack2(p.scale * co[j][0], p.scale * co[j][1]),
                                  pack2(p.scale * co[j][2], p.scale * co[j][3])};
                __builtin_amdgcn_raw_buffer_store_b64(ow, ro, ob + (uint32_t)(a * 16) * rsv + 32 * j, 0, 0);
            }
        }
    };
    // the pair of state tiles 2s, 2s+1 of column tile j times Pm, as one
    // 32-deep B operand
    auto sp_frag = [&](const float* pm, int j, int s) {
        const int g = (int)opaque((uint32_t)l) >> 4;
        const float4 m0 = ld4(pm + s * 32 + g * 8), m1 = ld4(pm + s * 32 + g * 8 + 4);
        const f32x4 a = {m0.x * S[j][2 * s][0], m0.y * S[j][2 * s][1], m0.z * S[j][2 * s][2],
                         m0.w * S[j][2 * s][3]};
        const f32x4 b = {m1.x * S[j][2 * s + 1][0], m1.y * S[j][2 * s + 1][1], m1.z * S[j][2 * s + 1][2],
                         m1.w * S[j][2 * s + 1][3]};
        return Mf::F32{__builtin_shufflevector(Mf::pack16(a).v, Mf::pack16(b).v, 0, 1, 2, 3, 4, 5, 6, 7)};
    };
    if constexpr (QN) __syncthreads();
    __syncthreads();
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int par = ch & 1;
        // ======================= segment 1 =======================
        // with two tiles per consumer (DVT 64) the consumers' segment-1 work is
        // as long as the producers', and they share the raised priority
        __builtin_amdgcn_s_setprio(NT > 1 ? 2 : 0);
        {
            const int lx = (int)opaque((uint32_t)l);  // addresses recomputed per chunk
            const int ln = lx & 15, lg = lx >> 4;
            if constexpr (CKPT) store_state(ckpt_at(ch));
            if (ch > 0) c_out(ch - 1);
            const bf16_t* kr_b = reinterpret_cast<const bf16_t*>(buf(par, L::bKr));
            const bf16_t* qr_b = reinterpret_cast<const bf16_t*>(buf(par, L::bQr));
            const float* beta = reinterpret_cast<const float*>(buf(par, L::bBeta));
            const float* vec = reinterpret_cast<const float*>(buf(par, L::bVec));
            const bf16_t* vt_b = reinterpret_cast<const bf16_t*>(buf(par, L::bVT));
            Mf::F32 fs[NT][DK / 32];
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int s = 0; s < DK / 32; ++s) fs[j][s] = sp_frag(vec, j, s);
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4 cx[NT], co[NT];
#pragma unroll
                for (int j = 0; j < NT; ++j) cx[j] = co[j] = zero4();
#pragma unroll
                for (int s = 0; s < DK / 32; ++s) {
                    const auto fk = Mf::ld32(frag_at(kr_b, a, s, ln, lg));
                    const auto fq = Mf::ld32(frag_at(qr_b, a, s, ln, lg));
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        cx[j] = Mf::k32(fk, fs[j][s], cx[j]);
                        co[j] = Mf::k32(fs[j][s], fq, co[j]);  // transposed, as c_out takes it
                    }
                }
                const float4 b4 = ld4(beta + a * 16 + lg * 4);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const uint2 v4 = *reinterpret_cast<const uint2*>(
                        vt_b + ((cj * NT + j) * 16 + ln) * L::LDV + a * 16 + lg * 4);
                    // beta_r (v_r - (Kr Pm S0)_r); rows past the end have v = beta = 0
                    Y[j][a][0] = b4.x * (lo_f(v4.x) - cx[j][0]);
                    Y[j][a][1] = b4.y * (hi_f(v4.x) - cx[j][1]);
                    Y[j][a][2] = b4.z * (lo_f(v4.y) - cx[j][2]);
                    Y[j][a][3] = b4.w * (hi_f(v4.y) - cx[j][3]);
                    OI[j][a] = co[j];
                }
            }
        }
        __syncthreads();
        // ======================= segment 2 =======================
        __builtin_amdgcn_s_setprio(3);
        {
            const int lx = (int)opaque((uint32_t)l);  // addresses recomputed per chunk
            const int ln = lx & 15, lg = lx >> 4;
            const bf16_t* lo_b = reinterpret_cast<const bf16_t*>(buf(par, L::bLo));
            const float* vec = reinterpret_cast<const float*>(buf(par, L::bVec));
            // U_a = D_a (Y_a - sum_{b<a} L_ab U_b); lo_b holds -L_ab.  All
            // fragments are read before the chains start, so no step of a
            // chain waits for LDS.
            Mf::F16 fl[6], fd[4];
#pragma unroll
            for (int i = 0; i < 6; ++i) fl[i] = Mf::ld16(lo_b + i * BLK + ln * LDB + lg * 4);
#pragma unroll
            for (int a = 0; a < 4; ++a) fd[a] = Mf::ld16(sD + a * BLK + ln * LDB + lg * 4);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int a = 0; a < 4; ++a) {
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    f32x4 acc = Y[j][a];
#pragma unroll
                    for (int b = 0; b < a; ++b) acc = Mf::k16(fl[a * (a - 1) / 2 + b], UP[j][b], acc);
                    UP[j][a] = Mf::pack16(Mf::k16(fd[a], Mf::pack16(acc), zero4()));
                }
            }
            // S <- Pn*S0 + (Pn/Pm) (Kc^T U); blocks 2s, 2s+1 of U form k-step s
            Mf::F32 fu[NT][2];
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    fu[j][s].v = __builtin_shufflevector(UP[j][2 * s].v, UP[j][2 * s + 1].v, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 acc[NT];
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[j] = zero4();
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const auto fkt = Mf::ld32(sKcT + (ct * 16 + ln) * LDC + s * 32 + lg * 8);
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[j] = Mf::k32(fkt, fu[j][s], acc[j]);
                }
                const int c0 = state_ch(ct, lg, 0);
                const float4 pn = ld4(vec + DK + c0);
                const float4 pnm = ld4(vec + 2 * DK + c0);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    S[j][ct][0] = pn.x * S[j][ct][0] + pnm.x * acc[j][0];
                    S[j][ct][1] = pn.y * S[j][ct][1] + pnm.y * acc[j][1];
                    S[j][ct][2] = pn.z * S[j][ct][2] + pnm.z * acc[j][2];
                    S[j][ct][3] = pn.w * S[j][ct][3] + pnm.w * acc[j][3];
                }
            }
        }
        __syncthreads();
    }

    if (nch > 0) c_out(nch - 1);
    if (finish()) {
        redo();
        return;
    }
    if constexpr (CKPT) store_state(ckpt_at(nch));
    if (p.sT) store_state(p.sT + sbase);
}

template <int DK, int DVT, int GATE, int FE, bool CKPT = false>
static hipError_t launch_g(const KParams& p, hipStream_t stream) {
    using Lay = Lay6<DK, DVT, (FE & FUSE_QK_L2NORM) != 0>;
    static const hipError_t attr = hipFuncSetAttribute(
        (const void*)chunk_fwd_bf16_kernel<DK, DVT, GATE, FE, CKPT>,
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    const long grid = 8L * p.njt_all * ((p.units + 7) / 8);
    hipLaunchKernelGGL((chunk_fwd_bf16_kernel<DK, DVT, GATE, FE, CKPT>), dim3((unsigned)grid),
                       dim3(Lay::NTH), Lay::bytes, stream, p);
    return hipGetLastError();
}

// the front-end instantiations: gate logits and q/k normalisation (beta
// logits are a run-time flag)
template <int DK, int DVT, int GATE>
static hipError_t launch_fe(const KParams& p, hipStream_t stream) {
    const bool gl = (p.fuse & FUSE_GATE_LOGITS) != 0, qn = (p.fuse & FUSE_QK_L2NORM) != 0;
    if constexpr (GATE == 2) {
        return qn ? launch_g<DK, DVT, 2, FUSE_QK_L2NORM>(p, stream) : launch_g<DK, DVT, 2, 0>(p, stream);
    } else {
        if (gl && qn) return launch_g<DK, DVT, GATE, FUSE_GATE_LOGITS | FUSE_QK_L2NORM>(p, stream);
        if (gl) return launch_g<DK, DVT, GATE, FUSE_GATE_LOGITS>(p, stream);
        if (qn) return launch_g<DK, DVT, GATE, FUSE_QK_L2NORM>(p, stream);
        return launch_g<DK, DVT, GATE, 0>(p, stream);
    }
}

template <int DK, int DVT>
static hipError_t launch_t(const KParams& p, hipStream_t stream) {
    // the backward's forward: per-channel gate, no input preparation
    if (p.ckpt) return launch_g<DK, DVT, 0, 0, true>(p, stream);
    return p.gate == 0 ? launch_fe<DK, DVT, 0>(p, stream)
         : p.gate == 1 ? launch_fe<DK, DVT, 1>(p, stream) : launch_fe<DK, DVT, 2>(p, stream);
}

// value-column tile widths this kernel supports
bool chunk_bf16_supports(int dvt) { return dvt == 16 || dvt == 32 || dvt == 64; }

hipError_t launch_chunk_bf16(const KParams& p, int dk, int dvt, hipStream_t stream) {
    if (dk == 128)
        return dvt == 16 ? launch_t<128, 16>(p, stream)
             : dvt == 32 ? launch_t<128, 32>(p, stream) : launch_t<128, 64>(p, stream);
    return dvt == 16 ? launch_t<64, 16>(p, stream)
         : dvt == 32 ? launch_t<64, 32>(p, stream) : launch_t<64, 64>(p, stream);
}

}  // namespace kda
