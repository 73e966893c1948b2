// tg_device.hpp -- device-side helpers shared by the gfx950 kernels.
//
// The epilogue every fused kernel applies to its fp32 accumulator while it is
// still in registers ("Fusing an Epilogue", teenygrad docs, section "The shape
// of it"): v = acc * scale[k] + bias[k] (inference BatchNorm folded per output
// channel), then y = v * sigmoid(v) (SiLU), then one cast and one store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

typedef _Float16 f16;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Epilogue selector: FUSED applies BatchNorm + SiLU; IDENTITY stores the raw
// convolution (the first kernel of the unfused, split and training-mode
// paths); RELU, GELU and BN apply BatchNorm and then max(v, 0), the exact
// GELU v * Phi(v), or nothing -- the other elementwise work "Fusing an
// Epilogue" (section "What an epilogue is") lists as belonging in the
// producer's epilogue (activations, bias adds, scaling).
enum Epilogue { EPI_FUSED = 0, EPI_IDENTITY = 1, EPI_RELU = 2, EPI_GELU = 3, EPI_BN = 4 };
constexpr int kNumEpilogues = 5;

// Instantiate X(E) for the run-time epilogue `epi` (one of the above).
#define TG_EPI_DISPATCH(epi, X)                               \
    do {                                                      \
        switch (epi) {                                        \
            case ::tg::EPI_IDENTITY: X(::tg::EPI_IDENTITY); break; \
            case ::tg::EPI_RELU: X(::tg::EPI_RELU); break;     \
            case ::tg::EPI_GELU: X(::tg::EPI_GELU); break;     \
            case ::tg::EPI_BN: X(::tg::EPI_BN); break;         \
            default: X(::tg::EPI_FUSED); break;               \
        }                                                     \
    } while (0)

// sigmoid(v) = 1 / (1 + e^-v), with e^-v = 2^(-v * log2 e) on the hardware
// exp2 (v_exp_f32) and the hardware reciprocal (v_rcp_f32). For v below about
// -88 the exponential is +inf and the reciprocal 0, so silu(v) is -0 (no NaN);
// for large v the exponential underflows to 0 and silu(v) = v.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float silu_f32(float v) {
    float e = __builtin_amdgcn_exp2f(-v * kLog2e);
    return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// The fused epilogue in five VALU operations. Kernels load each channel's
// BatchNorm scale and bias once and keep s2 = scale*log2(e), b2 =
// bias*log2(e) (epi_consts); then, with v = acc*scale + bias,
//   v2 = fma(acc, s2, b2)            = v * log2(e)
//   e  = 2^(-v2)                     = e^(-v)        (negation is free)
//   d  = fma(e, log2(e), log2(e))    = (1 + e^(-v)) * log2(e)
//   y  = v2 * rcp(d)                 = v / (1 + e^(-v)) = v * sigmoid(v).
// The identity epilogue (first kernel of the unfused baseline) returns acc.
// s2, b2 of output channel o (zero past C_out). The index is clamped instead
// of branching around the load, so all of a kernel's constant loads are in
// flight together and its prologue waits for one memory latency, not one per
// channel. The identity epilogue loads nothing.
// The other BatchNorm epilogues keep scale and bias as they are (epi_scale).
template <int EPI>
__device__ __forceinline__ float epi_scale(float c) {
    return EPI == EPI_FUSED ? c * kLog2e : (EPI == EPI_IDENTITY ? 0.0f : c);
}

template <int EPI>
__device__ __forceinline__ void epi_consts(const float* __restrict__ scale,
                                           const float* __restrict__ bias, int o, int C_out,
                                           float& s2, float& b2) {
    if (EPI == EPI_IDENTITY) {
        s2 = b2 = 0.0f;
        return;
    }
    const bool ok = o < C_out;
    const int oc = ok ? o : C_out - 1;
    const float s = scale[oc], b = bias[oc];
    s2 = ok ? epi_scale<EPI>(s) : 0.0f;
    b2 = ok ? epi_scale<EPI>(b) : 0.0f;
}

// GELU(v) = v * Phi(v) = v/2 * (1 + erf(v / sqrt 2)), with the device
// library's single-precision erf.
constexpr float kRsqrt2 = 0.70710678118654752f;

template <int EPI>
__device__ __forceinline__ float epilogue(float acc, float s2, float b2) {
    if (EPI == EPI_FUSED) {
        float v2 = __builtin_fmaf(acc, s2, b2);
        float e = __builtin_amdgcn_exp2f(-v2);
        float d = __builtin_fmaf(e, kLog2e, kLog2e);
        return v2 * __builtin_amdgcn_rcpf(d);
    }
    if (EPI == EPI_IDENTITY) return acc;
    const float v = __builtin_fmaf(acc, s2, b2);
    if (EPI == EPI_RELU) return v > 0.0f ? v : 0.0f;
    if (EPI == EPI_GELU) return 0.5f * v * (1.0f + erff(v * kRsqrt2));
    return v;  // EPI_BN
}

// fp8 output ("Fusing an Epilogue", section "What an epilogue is": casts to
// a narrower dtype belong in the epilogue): OCP E4M3, round to nearest even,
// with gfx950's v_cvt_pk_fp8_f32. Element e of y is then byte e. The kernels
// keep their fp16 output tiles and convert at the store; `out8` comes from
// the kernel arguments, so the branch is uniform and each store site issues
// exactly one store instruction either way.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2_t fp8x8(half8_t v) {
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[0], (float)v[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[2], (float)v[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[4], (float)v[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[6], (float)v[7], hi, true);
    return (u32x2_t){(unsigned)lo, (unsigned)hi};
}

// Residual add (the last elementwise step of a residual block, done in the
// producer's epilogue -- "Kernel Fusion", the passage on elementwise chains:
// bias, scale, activation, dropout mask and residual add fuse freely): the
// activated fp16 value plus the residual, added in fp32 and rounded once.
__device__ __forceinline__ half8_t res_add8(half8_t v, const _Float16* res, long long e) {
    const half8_t r = *(const half8_t*)(res + e);
    half8_t o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (_Float16)((float)v[i] + (float)r[i]);
    return o;
}

// Eight outputs from element e (a multiple of 8) of y; NT: non-temporal
// store. NT is a template parameter on purpose: with a run-time flag the
// compiler merges the two stores of an if/else into one and drops the
// non-temporal hint (measured: 25% slower on the 1x1 layer).
template <bool NT>
__device__ __forceinline__ void store_y8(_Float16* y, long long e, half8_t v, int out8,
                                         const void* res = nullptr) {
    if (res) v = res_add8(v, (const _Float16*)res, e);
    if (out8) {
        u32x2_t* p = (u32x2_t*)((unsigned char*)y + e);
        if constexpr (NT) __builtin_nontemporal_store(fp8x8(v), p);
        else *p = fp8x8(v);
    } else {
        half8_t* p = (half8_t*)(y + e);
        if constexpr (NT) __builtin_nontemporal_store(v, p);
        else *p = v;
    }
}

// One output, element e of y.
__device__ __forceinline__ void store_y1(_Float16* y, long long e, _Float16 v, int out8,
                                         const void* res = nullptr) {
    if (res) v = (_Float16)((float)v + (float)((const _Float16*)res)[e]);
    if (out8)
        ((unsigned char*)y)[e] =
            (unsigned char)(__builtin_amdgcn_cvt_pk_fp8_f32((float)v, 0.0f, 0, false) & 0xff);
    else
        y[e] = v;
}

template <typename T> __device__ __forceinline__ float to_f32(T v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return (T)v; }  // RNE

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8). Remap so that each XCD receives one contiguous range of logical
// tiles: neighbouring tiles (which share halo rows of x, or the same x rows
// for different channel tiles) then meet in the same L2. Bijective on
// [0, total) for any total.
__device__ __forceinline__ int xcd_contiguous_tile(int b, int total) {
    const int kXcds = 8;
    int xcd = b % kXcds, local = b / kXcds;
    int per = total / kXcds, rem = total % kXcds;
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Batch statistics (training-mode BatchNorm) of the kernels' epilogues.
//
// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15), left in every
// lane of the row: pairs, quads (quad permutes), then the other quad of the
// half row (half mirror) and the other half (mirror). Each step adds two
// values in either order, so all 16 lanes end with the same bits.
__device__ __forceinline__ float row_sum16(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)); // row_half_mirror
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)); // row_mirror
    return v;
}

// (n, mean, M2) of the union of two disjoint sets; (0, 0, 0) is the empty set.
__device__ __forceinline__ void chan_merge(double& n, double& mean, double& m2, double nb,
                                           double meanb, double m2b) {
    const double nt = n + nb;
    if (nt == 0.0) return;
    const double d = meanb - mean;
    const double f = nb / nt;
    mean = mean + d * f;
    m2 = m2 + m2b + d * d * n * f;
    n = nt;
}

}  // namespace tg
