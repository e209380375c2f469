// chunk_split.hip -- the chunk-wise forward of long dense sequences with few
// units, in two time segments that run at the same time.
//
// The token update of "Kimi Delta Attention", section "KDA 的更新式", is affine
// in the state: S_t = A_t S_{t-1} + b_t with A_t = (I - beta_t k_t k_t^T)
// Diag(alpha_t) and b_t = beta_t k_t v_t^T.  Over the second segment
// (tokens L0 .. T-1) of a sequence, started from any state X,
//   S_t = Phi_t X + R_t,   o_t = scale S_t^T q_t = X^T z_t + o^R_t,
// where Phi_t is the product of the segment's transitions so far (the same
// recurrence run from the identity with every value zero), z_t = scale
// Phi_t^T q_t its outputs, and R_t, o^R_t the recurrence from the zero state.
// None of them needs X, so the second segment's transition part (dk columns)
// and zero-start part (dv columns) run beside the first segment (from the
// caller's initial state); the first segment's final state Sm then gives the
// second segment's outputs, o_t = o^R_t + Sm^T z_t, and the final state,
// Phi_T Sm + R_T.  This is the chunk-parallel state passing of the kongchang
// page, section "硬件效率的优化策略", applied inside one sequence: with few
// (sequence, head) units the single pass leaves each unit's chain of chunks
// too long and its value slices too narrow, while here the first segment runs
// in 32-column slices and the second in 64-column ones, each cheaper per
// column than the 16-column slices the single pass needs to fill the chip.
//
// Outputs are those of the single pass up to rounding: z is stored in bf16 and
// Sm enters the output products as the sum of two bf16 parts (hi + lo, about
// 16 significant bits), with fp32 accumulation.
#include "chunk_common.h"

#include <mutex>

namespace kda {

namespace {
constexpr int SD = 128;  // dk = dv of the split path
// second-segment tokens per output block: 36 tiles of 16, which deal the long-context
// workload's blocks (32 units x 48) to 256 compute units, three at a time, in two whole rounds
constexpr int OUT_TOKENS = 576;
}  // namespace

// Final states: sT[u] = Phi[u] Sm[u] + R[u] (fp32, 128 x 128 per unit).
// State block (u, cb) forms columns 16 cb .. 16 cb + 15; thread t row t / 2 and
// eight of those columns.  Sm and sT may not overlap, but sT may be the
// caller's initial state (read by the first segment, which has ended).
__device__ __forceinline__ void split_state_block(const float* __restrict__ phi,
                                                  const float* __restrict__ sm,
                                                  const float* __restrict__ r,
                                                  float* __restrict__ sT, int u, int cb) {
    __shared__ float tile[SD][16];
    const size_t ub = (size_t)u * SD * SD;
    const int c0 = cb * 16;
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = t + 256 * i;  // element (row e / 16, column e % 16) of the tile
        tile[e >> 4][e & 15] = sm[ub + (size_t)(e >> 4) * SD + c0 + (e & 15)];
    }
    __syncthreads();
    const int row = t >> 1, cc = (t & 1) * 8;
    const float4* prow = reinterpret_cast<const float4*>(phi + ub + (size_t)row * SD);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int m4 = 0; m4 < SD / 4; ++m4) {
        const float4 a = prow[m4];
        const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(av[i], tile[4 * m4 + i][cc + e], acc[e]);
    }
    const size_t ob = ub + (size_t)row * SD + c0 + cc;
#pragma unroll
    for (int e = 0; e < 8; ++e) sT[ob + e] = acc[e] + r[ob + e];
}

// Second-segment outputs: o_t += Sm^T z_t, in place over o^R_t.
// Output block (u, tb): unit u = seq * H + h, second-segment tokens
// tb * OUT_TOKENS .. of it, in tiles of 16 tokens.  Wave w owns value columns
// 32 w .. 32 w + 31 as two 16-row tiles of C^T = Sm^T Z^T (rows: value
// columns j, columns: tokens), so that a lane holds four adjacent value
// columns of one token and writes them with one 8-byte store.  The A
// fragments (Sm^T, split in bf16 hi and lo parts, each with its own
// accumulator chain) stay in registers for all the block's tokens.  Each z
// tile (16 rows of 256 bytes) is loaded once per block, one 16-byte word per
// thread, and handed to the waves through LDS (rows 288 bytes apart, so the
// fragment reads are free of bank conflicts); z and o^R are loaded OUT_AHEAD
// tiles before their use.
//   o: the caller's output, rows seq * T + L0 + tau; z: rows seq * T + tau.
constexpr int OUT_AHEAD = 6;
constexpr int ZPITCH = SD + 16;  // bf16 elements per LDS row of a z tile
__device__ __forceinline__ void split_out_block(const float* __restrict__ sm,
                                                const bf16_t* __restrict__ z,
                                                bf16_t* __restrict__ o, int H, int T, int L0,
                                                int L1, int u, int tb) {
    using Mf = Mma<bf16_t>;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __shared__ __align__(16) bf16_t zs[2][16 * ZPITCH];
    const int seq = u / H, h = u % H;
    const int tb0 = tb * OUT_TOKENS;
    const int t = threadIdx.x;
    const int w = t >> 6, l = t & 63, ln = l & 15, lg = l >> 4;
    const float* smu = sm + (size_t)u * SD * SD;

    Mf::F32 ahi[2][4], alo[2][4];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
        const int j = 32 * w + 16 * jt + ln;  // value column: row of Sm^T
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = smu[(size_t)(32 * s + 8 * lg + e) * SD + j];
                const bf16_t hi = (bf16_t)x;
                ahi[jt][s].v[e] = hi;
                alo[jt][s].v[e] = (bf16_t)(x - to_f32(hi));
            }
        }
    }

    const size_t rs = (size_t)H * SD;  // elements per token row
    const int zr = t >> 4, zc = t & 15;  // this thread's row and 16-byte word of a z tile
    const bf16_t* zu = z + (size_t)seq * T * rs + (size_t)h * SD + 8 * zc;
    bf16_t* ou = o + ((size_t)seq * T + L0) * rs + (size_t)h * SD + 32 * w + 4 * lg;
    const int tend = min(L1, tb0 + OUT_TOKENS);
    const int ntiles = (tend - tb0 + 15) / 16;

    u32x4 zw[OUT_AHEAD];       // z words in flight
    bf16x4 rw[OUT_AHEAD][2];   // o^R of the lane's token, both column tiles
    auto load = [&](int n, int slot) __attribute__((always_inline)) {
        const int tau0 = tb0 + 16 * n;
        const int tz = tau0 + zr, to = tau0 + ln;
        if (tz < tend) zw[slot] = *reinterpret_cast<const u32x4*>(zu + (size_t)tz * rs);
        else zw[slot] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            if (to < tend) {
                rw[slot][jt] = *reinterpret_cast<const bf16x4*>(ou + (size_t)to * rs + 16 * jt);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) rw[slot][jt][e] = (bf16_t)0.f;
            }
        }
    };
#pragma unroll
    for (int k = 0; k < OUT_AHEAD; ++k) load(k, k);

    for (int n0 = 0; n0 < ntiles; n0 += OUT_AHEAD) {
#pragma unroll
        for (int k = 0; k < OUT_AHEAD; ++k) {
            const int n = n0 + k;
            if (n < ntiles) {  // the same for every thread of the block
                bf16_t* zb = zs[n & 1];
                *reinterpret_cast<u32x4*>(zb + zr * ZPITCH + 8 * zc) = zw[k];
                __syncthreads();
                Mf::F32 bz[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) bz[s] = Mf::ld32(zb + ln * ZPITCH + 32 * s + 8 * lg);
                const int tau = tb0 + 16 * n + ln;
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    f32x4 a0, a1 = zero4();
#pragma unroll
                    for (int e = 0; e < 4; ++e) a0[e] = to_f32(rw[k][jt][e]);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        a0 = Mf::k32(ahi[jt][s], bz[s], a0);
                        a1 = Mf::k32(alo[jt][s], bz[s], a1);
                    }
                    if (tau < tend) {
                        bf16x4 r4;
#pragma unroll
                        for (int e = 0; e < 4; ++e) r4[e] = (bf16_t)(a0[e] + a1[e]);
                        *reinterpret_cast<bf16x4*>(ou + (size_t)tau * rs + 16 * jt) = r4;
                    }
                }
                if (n + OUT_AHEAD < ntiles) load(n + OUT_AHEAD, k);
            }
        }
    }
}

// The last step of a call, one launch: blocks (u, y) with y < nblk form
// second-segment outputs, y = nblk + cb (when the final state is wanted) the
// final state's columns 16 cb ...
__global__ __launch_bounds__(256) void split_finish_kernel(const float* __restrict__ phi,
                                                           const float* __restrict__ sm,
                                                           const float* __restrict__ r,
                                                           float* __restrict__ sT,
                                                           const bf16_t* __restrict__ z,
                                                           bf16_t* __restrict__ o, int H, int T,
                                                           int L0, int L1, int nblk) {
    if ((int)blockIdx.y < nblk)
        split_out_block(sm, z, o, H, T, L0, L1, blockIdx.x, blockIdx.y);
    else
        split_state_block(phi, sm, r, sT, blockIdx.x, blockIdx.y - nblk);
}

namespace {

// Two more streams per device, the event that forks work onto them and the
// two that join them back, made once per device; one lock covers their making
// and every call's enqueue sequence, so that concurrent callers never
// interleave their records and waits on the shared events.
struct Aux {
    hipStream_t s[2] = {nullptr, nullptr};
    hipEvent_t fork = nullptr, join[2] = {nullptr, nullptr};
};
constexpr int kMaxDevices = 64;
std::mutex g_aux_mu;
Aux g_aux[kMaxDevices];

// (called with g_aux_mu held)
hipError_t aux_for(hipStream_t stream, Aux** out) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    Aux& a = g_aux[dev];
    if (!a.s[0]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        Aux n;
        e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
        for (int i = 0; i < 2 && e == hipSuccess; ++i) {
            e = hipStreamCreateWithFlags(&n.s[i], hipStreamNonBlocking);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join[i], hipEventDisableTiming);
        }
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        a = n;
    }
    *out = &a;
    return hipSuccess;
}

template <typename T>
const T* shift(const T* p, size_t bytes) {
    return p ? reinterpret_cast<const T*>(reinterpret_cast<const unsigned char*>(p) + bytes) : p;
}

}  // namespace

hipError_t launch_chunk_split(const ChunkArgs& a, void* ws, hipStream_t stream) {
    const SplitPlan sp = chunk_split_plan(a.B, a.T, a.H, a.dk, a.dv);
    if (sp.bytes == 0 || !ws) return hipErrorInvalidValue;
    const int units = a.B * a.H;
    unsigned char* w8 = static_cast<unsigned char*>(ws);
    float* sm = reinterpret_cast<float*>(w8 + sp.off_sm);
    float* phi = reinterpret_cast<float*>(w8 + sp.off_phi);
    float* rr = reinterpret_cast<float*>(w8 + sp.off_r);
    bf16_t* zz = reinterpret_cast<bf16_t*>(w8 + sp.off_z);

    KParams p0;
    p0.q = a.q; p0.k = a.k; p0.v = a.v; p0.alpha = a.alpha; p0.beta = a.beta; p0.s0 = a.s0;
    p0.o = a.o; p0.sT = sm; p0.cu_seqlens = nullptr; p0.order = nullptr;
    p0.B = a.B; p0.T = a.T; p0.H = a.H; p0.dv = a.dv;
    p0.units = units;
    p0.njt_all = a.dv / 32;
    p0.gate = a.gate;
    p0.fuse = a.fuse;
    p0.scale = a.scale;
    p0.t_len = sp.l0;

    // the second segment: every input row pointer moved L0 tokens on
    const size_t L0 = (size_t)sp.l0, H = (size_t)a.H;
    const size_t ges = (a.fuse & FUSE_GATE_LOGITS) ? 2 : 4;
    const size_t gw = a.gate == 0 ? (size_t)a.dk : a.gate == 1 ? 1 : 0;
    KParams pr = p0;  // the zero-start part: o^R into the caller's rows, R_T
    pr.q = shift(static_cast<const unsigned char*>(a.q), L0 * H * a.dk * 2);
    pr.k = shift(static_cast<const unsigned char*>(a.k), L0 * H * a.dk * 2);
    pr.v = shift(static_cast<const unsigned char*>(a.v), L0 * H * a.dv * 2);
    pr.alpha = shift(static_cast<const unsigned char*>(a.alpha), L0 * H * gw * ges);
    pr.beta = shift(a.beta, L0 * H * 4);
    pr.s0 = nullptr;
    pr.o = static_cast<unsigned char*>(a.o) + L0 * H * a.dv * 2;
    pr.sT = rr;
    pr.njt_all = a.dv / 64;
    pr.t_len = sp.l1;
    KParams pp = pr;  // the transition part: z and Phi_T
    pp.ident = true;
    pp.o = zz;
    pp.sT = phi;

    hipError_t e;
    {
        std::lock_guard<std::mutex> lock(g_aux_mu);
        Aux* ax = nullptr;
        if ((e = aux_for(stream, &ax)) != hipSuccess) return e;
        if ((e = hipEventRecord(ax->fork, stream)) != hipSuccess) return e;
        for (int i = 0; i < 2; ++i)
            if ((e = hipStreamWaitEvent(ax->s[i], ax->fork, 0)) != hipSuccess) return e;
        if ((e = launch_chunk_bf16(p0, a.dk, 32, stream)) != hipSuccess) return e;
        if ((e = launch_chunk_bf16(pr, a.dk, 64, ax->s[0])) != hipSuccess) return e;
        if ((e = launch_chunk_bf16(pp, a.dk, 64, ax->s[1])) != hipSuccess) return e;
        for (int i = 0; i < 2; ++i) {
            if ((e = hipEventRecord(ax->join[i], ax->s[i])) != hipSuccess) return e;
            if ((e = hipStreamWaitEvent(stream, ax->join[i], 0)) != hipSuccess) return e;
        }
    }
    const int nblk = (sp.l1 + OUT_TOKENS - 1) / OUT_TOKENS;
    hipLaunchKernelGGL(split_finish_kernel, dim3((unsigned)units, nblk + (a.sT ? SD / 16 : 0)),
                       dim3(256), 0, stream, phi, sm, rr, a.sT, zz, static_cast<bf16_t*>(a.o),
                       a.H, a.T, sp.l0, sp.l1, nblk);
    return hipGetLastError();
}

}  // namespace kda
