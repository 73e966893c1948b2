// scalar.hip -- conv2d_bn_silu_scalar: one output element per lane.
//
// "Fusing an Epilogue" (teenygrad docs), section "Three kernels for one
// operation": the scalar kernel has no setup cost and serves small shapes;
// here it is also the kernel that serves every shape and both dtypes.
//
// Lane -> (n, p, q, k) with k fastest, so the C_out lanes that share an
// output pixel read the same x values (one fetch serves them all) and the y
// stores of a wavefront are contiguous in NHWC.
#include <type_traits>

#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {

template <typename T, int EPI>
__global__ __launch_bounds__(256) void conv2d_bn_silu_scalar(
    const T* __restrict__ x, const T* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, T* __restrict__ y, ConvGeom g, int total) {
    // 64-bit before the comparison: with total close to 2^31 the last
    // block's lanes would overflow an int.
    const long long lidx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (lidx >= total) return;
    const int idx = (int)lidx;
    int k = idx % g.C_out;
    int pix = idx / g.C_out;
    int q = pix % g.Q;
    int t = pix / g.Q;
    int p = t % g.P;
    int n = t / g.P;
    int h0 = p * g.stride - g.pad, w0 = q * g.stride - g.pad;
    float acc = 0.0f;
    for (int r = 0; r < g.kh; ++r) {
        int ih = h0 + r;
        if ((unsigned)ih >= (unsigned)g.H) continue;
        for (int s = 0; s < g.kw; ++s) {
            int iw = w0 + s;
            if ((unsigned)iw >= (unsigned)g.W) continue;
            const T* xp = x + ((n * g.H + ih) * g.W + iw) * g.C_in;
            const T* wp = w + ((k * g.kh + r) * g.kw + s) * g.C_in;
            for (int c = 0; c < g.C_in; ++c) acc = __builtin_fmaf(to_f32(xp[c]), to_f32(wp[c]), acc);
        }
    }
    float sc, bi;
    epi_consts<EPI>(scale, bias, k, g.C_out, sc, bi);
    const T v = from_f32<T>(epilogue<EPI>(acc, sc, bi));
    if constexpr (std::is_same<T, f16>::value)
        store_y1(y, idx, v, g.out8, g.res);
    else
        y[idx] = g.res ? v + ((const T*)g.res)[idx] : v;
}

hipError_t launch_scalar(const ConvGeom& g, bool f32, int epi, const void* x, const void* w,
                         const float* scale, const float* bias, void* y, hipStream_t s) {
    const int total = g.M * g.C_out;  // < 2^31, checked at plan time
    dim3 grid((unsigned)(((long long)total + 255) / 256)), block(256);
#define TG_S32(E)                                                                \
    hipLaunchKernelGGL((conv2d_bn_silu_scalar<float, E>), grid, block, 0, s,       \
                       (const float*)x, (const float*)w, scale, bias, (float*)y, g, total)
#define TG_S16(E)                                                                \
    hipLaunchKernelGGL((conv2d_bn_silu_scalar<f16, E>), grid, block, 0, s,         \
                       (const f16*)x, (const f16*)w, scale, bias, (f16*)y, g, total)
    if (f32)
        TG_EPI_DISPATCH(epi, TG_S32);
    else
        TG_EPI_DISPATCH(epi, TG_S16);
#undef TG_S16
#undef TG_S32
    return hipGetLastError();
}

}  // namespace tg
