// kda_device.h -- gfx950 device helpers shared by the libkda kernels:
// bf16 <-> fp32 conversion and thin wrappers over the CDNA4 matrix-core
// (MFMA) instructions with one fragment convention for bf16 and fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(uint32_t(__builtin_bit_cast(uint16_t, x)) << 16);
}

// The logistic function 1 / (1 + e^-z), with e^-z = 2^(-z log2 e) taken by the
// hardware base-2 exponential and the division by its reciprocal (about two
// ulp); z -> -inf gives 0, z -> +inf gives 1.
__device__ __forceinline__ float sigmoid_f(float z) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}
// 1 / sqrt(ss + 1e-6): the scale that L2-normalises a vector with squared norm
// ss (a zero vector stays zero)
__device__ __forceinline__ float inv_norm(float ss) { return __builtin_amdgcn_rsqf(ss + 1e-6f); }

// in-kernel input preparation (kda_fuse_flag bits)
constexpr int FUSE_GATE_LOGITS = 1, FUSE_BETA_LOGITS = 2, FUSE_QK_L2NORM = 4;

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    return (bf16_t)x;  // v_cvt_pk_bf16_f32: round to nearest even
}

// ---------------------------------------------------------------------------
// Matrix-core tiles.  All products here are 16x16 output tiles with fp32
// accumulation, in the CDNA 16x16 layout: lane l holds rows 4*(l/16)+0..3 of
// column l%16 (an f32x4).
//
// Operand fragments use one k-convention for both element types: lane l
// supplies row (A) / column (B) l%16 and a run of consecutive k indices
// selected by its lane group g = l/16.  For a k-step of 32 the run is
// k = 8g..8g+7; for a k-step of 16 it is k = 4g..4g+3.  bf16 maps a step onto
// one v_mfma_f32_16x16x32_bf16 (or 16x16x16_bf16); fp32 splits it into 8 (or
// 4) v_mfma_f32_16x16x4_f32 whose i-th instruction takes element i of every
// lane's run.  Because A and B follow the same rule the contraction covers
// every k exactly once whatever order the hardware sums lane groups in.
// ---------------------------------------------------------------------------
template <typename Top>
struct Mma;

template <>
struct Mma<bf16_t> {
    struct F32 { bf16x8 v; };  // 8 k-values
    struct F16 { bf16x4 v; };  // 4 k-values
    static __device__ __forceinline__ F32 ld32(const bf16_t* p) {
        return F32{*reinterpret_cast<const bf16x8*>(p)};
    }
    static __device__ __forceinline__ F16 ld16(const bf16_t* p) {
        return F16{*reinterpret_cast<const bf16x4*>(p)};
    }
    static __device__ __forceinline__ F16 pack16(f32x4 c) {
        // two paired conversions (v_cvt_pk_bf16_f32), not four single ones
        bf16x2v lo, hi;
        lo[0] = (bf16_t)c[0]; lo[1] = (bf16_t)c[1];
        hi[0] = (bf16_t)c[2]; hi[1] = (bf16_t)c[3];
        typedef unsigned u2v __attribute__((ext_vector_type(2)));
        u2v w = {__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
        return F16{__builtin_bit_cast(bf16x4, w)};
    }
    static __device__ __forceinline__ f32x4 k32(F32 a, F32 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 k16(F16 a, F16 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a.v),
                                                        __builtin_bit_cast(short4v, b.v), c,
                                                        0, 0, 0);
    }
    // store 4 consecutive elements (one C-layout column run) to LDS
    static __device__ __forceinline__ void st4(bf16_t* p, f32x4 c) {
        bf16x4 h;
        h[0] = (bf16_t)c[0]; h[1] = (bf16_t)c[1]; h[2] = (bf16_t)c[2]; h[3] = (bf16_t)c[3];
        *reinterpret_cast<bf16x4*>(p) = h;
    }
};

template <>
struct Mma<float> {
    struct F32 { float4 lo, hi; };
    struct F16 { float4 v; };
    static __device__ __forceinline__ F32 ld32(const float* p) {
        return F32{reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
    }
    static __device__ __forceinline__ F16 ld16(const float* p) {
        return F16{*reinterpret_cast<const float4*>(p)};
    }
    static __device__ __forceinline__ F16 pack16(f32x4 c) {
        return F16{make_float4(c[0], c[1], c[2], c[3])};
    }
    static __device__ __forceinline__ f32x4 k32(F32 a, F32 b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ f32x4 k16(F16 a, F16 b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.x, b.v.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.y, b.v.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.z, b.v.z, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.w, b.v.w, c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ void st4(float* p, f32x4 c) {
        *reinterpret_cast<float4*>(p) = make_float4(c[0], c[1], c[2], c[3]);
    }
};

__device__ __forceinline__ f32x4 zero4() {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

}  // namespace kda
