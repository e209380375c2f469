// peaks.hip -- what one MI355X reaches on the two resources the chunk-wise
// forward is measured against: HBM bandwidth (a streaming copy and a
// read-only stream) and dense bf16 matrix-core throughput (independent
// chains of v_mfma_f32_16x16x32_bf16 on every SIMD).  Measurement kernels for
// the benchmark, built into their own library (libkda_peaks.so); nothing of
// the KDA path uses them.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte words in flight per thread and iteration

// dst[i] = src[i] over n 16-byte words; each thread moves kUnroll words per
// iteration, kUnroll * grid threads apart, so every load of an iteration is
// issued before the first store.
__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, size_t n) {
    const size_t nthr = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += nthr * kUnroll) {
        u32x4 w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t j = i + u * nthr;
            if (j < n) w[u] = src[j];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t j = i + u * nthr;
            if (j < n) __builtin_nontemporal_store(w[u], &dst[j]);
        }
    }
}

// Reads n 16-byte words; the XOR of everything a thread read is stored only if
// it equals `key` (which the caller picks so that it practically never does),
// so the loads stay live while the kernel writes next to nothing.
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, size_t n,
                                                        uint32_t key, uint32_t* __restrict__ sink) {
    const size_t nthr = (size_t)gridDim.x * kThreads;
    const size_t tid = (size_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t x = 0;
    for (size_t i = tid; i < n; i += nthr * kUnroll) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t j = i + u * nthr;
            if (j < n) {
                const u32x4 w = src[j];
                x ^= w[0] ^ w[1] ^ w[2] ^ w[3];
            }
        }
    }
    if (x == key) sink[tid] = x;
}

// Each wave runs kChains independent accumulator chains of `iters` bf16
// 16x16x32 matrix-core products (2 * 16 * 16 * 32 flops each); the sums are
// stored only if they equal `key`.
constexpr int kChains = 4;
__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, float key, float* __restrict__ sink) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.0f + 0.001f * (float)((threadIdx.x + e) & 7));
        b[e] = (__bf16)(0.5f - 0.001f * (float)((threadIdx.x * 3 + e) & 7));
    }
    f32x4 c[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
    if (s == key) sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Streaming copy of `bytes` (a multiple of 16, both pointers 16-byte aligned)
// from src to dst on `stream` with `blocks` workgroups of 256 threads.
// Returns a hipError_t code.
int kda_peak_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream) {
    if ((bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15) || blocks <= 0)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
    return (int)hipGetLastError();
}

// Read-only stream over `bytes` of src (as for kda_peak_copy); sink holds one
// uint32 per thread (blocks * 256) and is written at most where the XOR of a
// thread's words equals key.
int kda_peak_read(const void* src, size_t bytes, uint32_t key, uint32_t* sink, int blocks,
                  hipStream_t stream) {
    if ((bytes & 15) || ((uintptr_t)src & 15) || !sink || blocks <= 0)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(src), bytes / 16, key, sink);
    return (int)hipGetLastError();
}

// Matrix-core loop: blocks workgroups of 256 threads, each wave kChains chains
// of `iters` products; flops = blocks * 4 waves * kChains * iters * 16384.
// sink holds one float per thread (blocks * 256), written at most where a
// thread's sum equals key.
int kda_peak_mfma(int iters, float key, float* sink, int blocks, hipStream_t stream) {
    if (iters <= 0 || !sink || blocks <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(kThreads), 0, stream, iters, key, sink);
    return (int)hipGetLastError();
}

int kda_peak_mfma_chains(void) { return kChains; }

}  // extern "C"
