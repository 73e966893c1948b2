// tiled.hip -- conv2d_bn_silu_tiled: direct convolution tiled over the output
// spatial extent, for layers with few output channels.
//
// "Fusing an Epilogue" (teenygrad docs), section "Three kernels for one
// operation": the GEMM kernel wastes its tiles when output channels are few,
// so a kernel tiled over the output's spatial extent serves those shapes.
//
// One workgroup owns a band of R output rows of one image, all Q columns and
// all output channels. It stages the input rows the band needs (with zero
// padding materialised) and the filter bank in LDS: the input rows are
// contiguous in NHWC, so the staging loads are coalesced, and every input
// value is then read from LDS by each window that covers it instead of from
// memory. Work item = (output pixel, group of 8 output channels); consecutive
// lanes take consecutive channel groups and pixels, so the stores of a
// wavefront cover one contiguous run of y.
#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {

static constexpr int kTiledCG = 8;        // output channels per work item
static constexpr int kTiledMaxCout = 64;  // filter bank kept in LDS
static constexpr int kTiledLdsCap = 48 * 1024;

static inline int round_up(int a, int b) { return (a + b - 1) / b * b; }

static int tiled_lds_bytes(const ConvGeom& g, int R, int WPad) {
    int COP = round_up(g.C_out, kTiledCG);
    int RH = (R - 1) * g.stride + g.kh;
    return g.K * COP * 4 + round_up(RH * WPad * g.C_in * 2, 16);
}

bool tiled_plan(const ConvGeom& g, TiledCfg* out) {
    if (g.C_out > kTiledMaxCout) return false;
    int WPad = (g.Q - 1) * g.stride + g.kw;
    int R = g.P < 8 ? g.P : 8;
    while (R > 1 && tiled_lds_bytes(g, R, WPad) > kTiledLdsCap) --R;
    int bytes = tiled_lds_bytes(g, R, WPad);
    if (bytes > 64 * 1024) return false;
    out->R = R;
    out->WPad = WPad;
    out->lds_bytes = bytes;
    return true;
}

template <int EPI>
__global__ __launch_bounds__(256) void conv2d_bn_silu_tiled(
    const f16* __restrict__ x, const f16* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, f16* __restrict__ y, ConvGeom g, int R, int WPad) {
    extern __shared__ __attribute__((aligned(16))) float tiled_lds[];
    const int CG = kTiledCG;
    const int COP = (g.C_out + CG - 1) / CG * CG;
    const int G = COP / CG;
    const int bands = (g.P + R - 1) / R;
    const int n = blockIdx.x / bands, band = blockIdx.x - n * bands;
    const int p0 = band * R;
    const int rows_out = imin(R, g.P - p0);
    const int RH = (rows_out - 1) * g.stride + g.kh;
    const int ih0 = p0 * g.stride - g.pad, iw0 = -g.pad;
    const int tid = threadIdx.x;

    float* wl = tiled_lds;                 // [K][COP] fp32, zero beyond C_out
    f16* xl = (f16*)(tiled_lds + g.K * COP);  // [RH][WPad][C_in], zero outside the image

    for (int i = tid; i < g.K * COP; i += 256) {
        int k = i / COP, o = i - (i / COP) * COP;
        wl[i] = o < g.C_out ? (float)w[o * g.K + k] : 0.0f;
    }
    const int row_len = WPad * g.C_in;
    const f16* xn = x + n * g.H * g.W * g.C_in;
    for (int i = tid; i < RH * row_len; i += 256) {
        int rr = i / row_len, e = i - rr * row_len;
        int col = e / g.C_in, c = e - col * g.C_in;
        int ih = ih0 + rr, iw = iw0 + col;
        f16 v = (f16)0.0f;
        if ((unsigned)ih < (unsigned)g.H && (unsigned)iw < (unsigned)g.W)
            v = xn[(ih * g.W + iw) * g.C_in + c];
        xl[i] = v;
    }
    __syncthreads();

    const int items = rows_out * g.Q * G;
    for (int it = tid; it < items; it += 256) {
        int gi = it % G, pix = it / G;
        int q = pix % g.Q, pl = pix / g.Q;
        float acc[CG];
#pragma unroll
        for (int j = 0; j < CG; ++j) acc[j] = 0.0f;
        for (int r = 0; r < g.kh; ++r) {
            for (int s = 0; s < g.kw; ++s) {
                const f16* xp = xl + ((pl * g.stride + r) * WPad + q * g.stride + s) * g.C_in;
                const float* wp = wl + ((r * g.kw + s) * g.C_in) * COP + gi * CG;
                for (int c = 0; c < g.C_in; ++c) {
                    float xv = (float)xp[c];
                    float4_t w0 = *(const float4_t*)(wp + c * COP);
                    float4_t w1 = *(const float4_t*)(wp + c * COP + 4);
                    acc[0] = __builtin_fmaf(xv, w0[0], acc[0]);
                    acc[1] = __builtin_fmaf(xv, w0[1], acc[1]);
                    acc[2] = __builtin_fmaf(xv, w0[2], acc[2]);
                    acc[3] = __builtin_fmaf(xv, w0[3], acc[3]);
                    acc[4] = __builtin_fmaf(xv, w1[0], acc[4]);
                    acc[5] = __builtin_fmaf(xv, w1[1], acc[5]);
                    acc[6] = __builtin_fmaf(xv, w1[2], acc[6]);
                    acc[7] = __builtin_fmaf(xv, w1[3], acc[7]);
                }
            }
        }
        const int o0 = gi * CG;
        const int yp = ((n * g.P + p0 + pl) * g.Q + q) * g.C_out + o0;  // element of y
        if ((g.C_out & 7) == 0) {
            half8_t h;
#pragma unroll
            for (int j = 0; j < CG; ++j) {
                float sc, bi;
                epi_consts<EPI>(scale, bias, o0 + j, g.C_out, sc, bi);
                h[j] = (f16)epilogue<EPI>(acc[j], sc, bi);
            }
            store_y8<false>(y, yp, h, g.out8, g.res);
        } else {
#pragma unroll
            for (int j = 0; j < CG; ++j) {
                if (o0 + j < g.C_out) {
                    float sc, bi;
                    epi_consts<EPI>(scale, bias, o0 + j, g.C_out, sc, bi);
                    store_y1(y, yp + j, (f16)epilogue<EPI>(acc[j], sc, bi), g.out8, g.res);
                }
            }
        }
    }
}

hipError_t launch_tiled(const ConvGeom& g, const TiledCfg& c, int epi, const void* x,
                        const void* w, const float* scale, const float* bias, void* y,
                        hipStream_t s) {
    int bands = (g.P + c.R - 1) / c.R;
    dim3 grid(g.N * bands), block(256);
#define TG_T(E)                                                                        \
    hipLaunchKernelGGL(conv2d_bn_silu_tiled<E>, grid, block, c.lds_bytes, s, (const f16*)x, \
                       (const f16*)w, scale, bias, (f16*)y, g, c.R, c.WPad)
    TG_EPI_DISPATCH(epi, TG_T);
#undef TG_T
    return hipGetLastError();
}

}  // namespace tg
