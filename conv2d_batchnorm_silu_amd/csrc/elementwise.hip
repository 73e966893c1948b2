// elementwise.hip -- the BatchNorm fold, the two streaming kernels of the
// unfused three-kernel baseline, and the one streaming kernel of the split
// form (conv kernel, then BatchNorm+SiLU).
//
// Baseline ("Fusing an Epilogue", teenygrad docs, section "The problem"): the
// conv kernel writes t1, a batch-norm kernel reads t1 and writes t2, a SiLU
// kernel reads t2 and writes y. The conv stage reuses the fused kernels with
// an identity epilogue; these two kernels are the other stages. Both stream
// 16 bytes per lane when the tensor allows it and compute in fp32, like the
// fused epilogue, so the baseline differs from the fused path only in where
// t1 and t2 live.
#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {

// scale = gamma / sqrt(var + eps), bias = beta - mean * scale (fp32).
__global__ void bn_fold_kernel(const float* __restrict__ gamma, const float* __restrict__ beta,
                               const float* __restrict__ mean, const float* __restrict__ var,
                               float eps, int C, float* __restrict__ scale,
                               float* __restrict__ bias) {
    int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= C) return;
    float sc = gamma[c] / sqrtf(var[c] + eps);
    scale[c] = sc;
    bias[c] = beta[c] - mean[c] * sc;
}

// t2 = t1 * scale[c] + bias[c], c = element index mod C (channels-last).
template <typename T>
__global__ __launch_bounds__(256) void bn_apply_scalar(const T* __restrict__ t1,
                                                       const float* __restrict__ scale,
                                                       const float* __restrict__ bias,
                                                       T* __restrict__ t2, long long total, int C) {
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    int c = (int)(i % C);
    t2[i] = from_f32<T>(__builtin_fmaf(to_f32(t1[i]), scale[c], bias[c]));
}

__global__ __launch_bounds__(256) void bn_apply_f16x8(const half8_t* __restrict__ t1,
                                                      const float* __restrict__ scale,
                                                      const float* __restrict__ bias,
                                                      half8_t* __restrict__ t2, long long nvec,
                                                      int C) {
    long long j = (long long)blockIdx.x * 256 + threadIdx.x;
    if (j >= nvec) return;
    half8_t v = t1[j];
    int c = (int)((j * 8) % C);
    half8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o[e] = (f16)__builtin_fmaf((float)v[e], scale[c], bias[c]);
        c = (c + 1 == C) ? 0 : c + 1;
    }
    t2[j] = o;
}

// Channel counts that are multiples of 8: a lane's 8 halves are channels
// c0..c0+7 of one pixel, so its scale and bias come in two 16-byte loads each
// and the channel index is one 32-bit remainder per lane (element counts are
// below 2^31). MODE 0: BatchNorm only (t2 = t1*scale + bias, unfused
// baseline); MODE 1: BatchNorm + SiLU (split form).
// in and out may be the same buffer (training mode applies BatchNorm+SiLU to
// y in place): each lane reads its element before it writes it.
template <int MODE>
__global__ __launch_bounds__(256) void bn_c8_f16x8(const half8_t* in,
                                                   const float4_t* __restrict__ scale4,
                                                   const float4_t* __restrict__ bias4,
                                                   half8_t* out, unsigned nvec, unsigned cv) {
    const unsigned j = blockIdx.x * 256u + threadIdx.x;
    if (j >= nvec) return;
    const unsigned c4 = (j % cv) * 2u;
    const float4_t s0 = scale4[c4], s1 = scale4[c4 + 1], b0 = bias4[c4], b1 = bias4[c4 + 1];
    const half8_t v = in[j];
    half8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float s = e < 4 ? s0[e & 3] : s1[e & 3];
        const float b = e < 4 ? b0[e & 3] : b1[e & 3];
        if (MODE == 0)
            o[e] = (f16)__builtin_fmaf((float)v[e], s, b);
        else
            o[e] = (f16)epilogue<EPI_FUSED>((float)v[e], s * kLog2e, b * kLog2e);
    }
    out[j] = o;
}

template <typename T>
__global__ __launch_bounds__(256) void silu_apply_scalar(const T* __restrict__ t2, T* __restrict__ y,
                                                         long long total) {
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    y[i] = from_f32<T>(silu_f32(to_f32(t2[i])));
}

__global__ __launch_bounds__(256) void silu_apply_f16x8(const half8_t* __restrict__ t2,
                                                        half8_t* __restrict__ y, long long nvec) {
    long long j = (long long)blockIdx.x * 256 + threadIdx.x;
    if (j >= nvec) return;
    half8_t v = t2[j];
    half8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (f16)silu_f32((float)v[e]);
    y[j] = o;
}

// Split form ("Fusing an Epilogue", section "When not to fuse"; "Kernel
// Fusion", the passage on when fusion does not pay): the conv kernel writes t1, then
// this kernel applies the same fp32 epilogue as the fused kernels,
// y = silu(t1 * scale[c] + bias[c]), reading t1 once and writing y once.
// t1 and y may be the same buffer (training mode works in place).
template <typename T>
__global__ __launch_bounds__(256) void bn_silu_apply_scalar(const T* t1,
                                                            const float* __restrict__ scale,
                                                            const float* __restrict__ bias,
                                                            T* y, long long total, int C) {
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    int c = (int)(i % C);
    float s2, b2;
    epi_consts<EPI_FUSED>(scale, bias, c, C, s2, b2);
    y[i] = from_f32<T>(epilogue<EPI_FUSED>(to_f32(t1[i]), s2, b2));
}

__global__ __launch_bounds__(256) void bn_silu_apply_f16x8(const half8_t* t1,
                                                           const float* __restrict__ scale,
                                                           const float* __restrict__ bias,
                                                           half8_t* y, long long nvec, int C) {
    long long j = (long long)blockIdx.x * 256 + threadIdx.x;
    if (j >= nvec) return;
    half8_t v = t1[j];
    int c = (int)((j * 8) % C);
    half8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float s2, b2;
        epi_consts<EPI_FUSED>(scale, bias, c, C, s2, b2);
        o[e] = (f16)epilogue<EPI_FUSED>((float)v[e], s2, b2);
        c = (c + 1 == C) ? 0 : c + 1;
    }
    y[j] = o;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

hipError_t launch_bn_fold(const float* gamma, const float* beta, const float* mean,
                          const float* var, float eps, int C, float* scale, float* bias,
                          hipStream_t s) {
    hipLaunchKernelGGL(bn_fold_kernel, dim3((C + 255) / 256), dim3(256), 0, s, gamma, beta, mean,
                       var, eps, C, scale, bias);
    return hipGetLastError();
}

static bool c8_path(bool f32, const void* in, const float* scale, const float* bias,
                    const void* out, long long total, int C) {
    return !f32 && C % 8 == 0 && total % 8 == 0 && total < (1LL << 31) && aligned16(in) &&
           aligned16(out) && aligned16(scale) && aligned16(bias);
}

template <int MODE>
static void launch_c8(const void* in, const float* scale, const float* bias, void* out,
                      long long total, int C, hipStream_t s) {
    const unsigned nvec = (unsigned)(total / 8);
    hipLaunchKernelGGL(bn_c8_f16x8<MODE>, dim3((nvec + 255) / 256), dim3(256), 0, s,
                       (const half8_t*)in, (const float4_t*)scale, (const float4_t*)bias,
                       (half8_t*)out, nvec, (unsigned)(C / 8));
}

hipError_t launch_bn_apply(bool f32, const void* t1, const float* scale, const float* bias, void* t2,
                           long long total, int C, hipStream_t s) {
    if (c8_path(f32, t1, scale, bias, t2, total, C)) {
        launch_c8<0>(t1, scale, bias, t2, total, C, s);
    } else if (!f32 && total % 8 == 0 && aligned16(t1) && aligned16(t2)) {
        long long nvec = total / 8;
        hipLaunchKernelGGL(bn_apply_f16x8, dim3((unsigned)((nvec + 255) / 256)), dim3(256), 0, s,
                           (const half8_t*)t1, scale, bias, (half8_t*)t2, nvec, C);
    } else if (f32) {
        hipLaunchKernelGGL(bn_apply_scalar<float>, dim3((unsigned)((total + 255) / 256)), dim3(256),
                           0, s, (const float*)t1, scale, bias, (float*)t2, total, C);
    } else {
        hipLaunchKernelGGL(bn_apply_scalar<f16>, dim3((unsigned)((total + 255) / 256)), dim3(256),
                           0, s, (const f16*)t1, scale, bias, (f16*)t2, total, C);
    }
    return hipGetLastError();
}

hipError_t launch_bn_silu_apply(bool f32, const void* t1, const float* scale, const float* bias,
                                void* y, long long total, int C, hipStream_t s) {
    if (c8_path(f32, t1, scale, bias, y, total, C)) {
        launch_c8<1>(t1, scale, bias, y, total, C, s);
    } else if (!f32 && total % 8 == 0 && aligned16(t1) && aligned16(y)) {
        long long nvec = total / 8;
        hipLaunchKernelGGL(bn_silu_apply_f16x8, dim3((unsigned)((nvec + 255) / 256)), dim3(256), 0,
                           s, (const half8_t*)t1, scale, bias, (half8_t*)y, nvec, C);
    } else if (f32) {
        hipLaunchKernelGGL(bn_silu_apply_scalar<float>, dim3((unsigned)((total + 255) / 256)),
                           dim3(256), 0, s, (const float*)t1, scale, bias, (float*)y, total, C);
    } else {
        hipLaunchKernelGGL(bn_silu_apply_scalar<f16>, dim3((unsigned)((total + 255) / 256)),
                           dim3(256), 0, s, (const f16*)t1, scale, bias, (f16*)y, total, C);
    }
    return hipGetLastError();
}

hipError_t launch_silu_apply(bool f32, const void* t2, void* y, long long total, hipStream_t s) {
    if (!f32 && total % 8 == 0 && aligned16(t2) && aligned16(y)) {
        long long nvec = total / 8;
        hipLaunchKernelGGL(silu_apply_f16x8, dim3((unsigned)((nvec + 255) / 256)), dim3(256), 0, s,
                           (const half8_t*)t2, (half8_t*)y, nvec);
    } else if (f32) {
        hipLaunchKernelGGL(silu_apply_scalar<float>, dim3((unsigned)((total + 255) / 256)),
                           dim3(256), 0, s, (const float*)t2, (float*)y, total);
    } else {
        hipLaunchKernelGGL(silu_apply_scalar<f16>, dim3((unsigned)((total + 255) / 256)), dim3(256),
                           0, s, (const f16*)t2, (f16*)y, total);
    }
    return hipGetLastError();
}

}  // namespace tg
