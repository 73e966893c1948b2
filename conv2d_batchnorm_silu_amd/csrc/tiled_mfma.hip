// tiled_mfma.hip -- conv2d_bn_silu_tiled on the matrix cores: direct
// convolution tiled over the output's spatial extent, for layers whose whole
// reduction fits one MFMA step (K = kh*kw*C_in <= 32) and which have few
// output channels (C_out <= 32), such as an RGB stem.
//
// "Fusing an Epilogue" (teenygrad docs), section "Three kernels for one
// operation": the tiled kernel covers the output's spatial extent and serves
// layers with few output channels. On gfx950 the 16x16x32 fp16 MFMA does a
// 16-pixel x 16-channel x 32-deep block in one instruction, so the
// multiply-adds of such a layer cost almost nothing; what remains is moving
// x and y and the per-output epilogue.
//
// One workgroup owns a band of R output rows of one image:
//   1. The (R-1)*stride + kh input rows the band reads are copied into LDS
//      with zero columns for the padding. Those rows are contiguous in NHWC,
//      so the copy is a coalesced streaming read.
//   2. For each 16-pixel run of an output row, every lane gathers its
//      8 im2col values (pixel lane%16, k = 8*(lane/16) .. +7, k = (r, s, c)
//      flattened) from LDS into the MFMA column operand; the filter bank,
//      zero-padded to 32 taps, sits in the row operand for the whole kernel.
//   3. BatchNorm + SiLU on the accumulators; the fp16 results go to an LDS
//      copy of the band's output, which is contiguous in NHWC (R rows x Q
//      pixels x C_out channels), and the workgroup streams it out with
//      16-byte stores.
#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {

static constexpr int kTmLdsTarget = 40 * 1024;

// LDS input row: image data starts at the 16-byte aligned half DO (padding
// zeros just before it and just after it), rows are 16-byte multiples.
static __host__ __device__ inline int tm_data_off(const ConvGeom& g) {
    return (g.pad * g.C_in + 7) / 8 * 8;
}
static __host__ __device__ inline int tm_row_halves(const ConvGeom& g) {
    int halves = tm_data_off(g) + g.W * g.C_in + g.pad * g.C_in;
    return (halves + 7) / 8 * 8;
}

static int tm_lds_bytes(const ConvGeom& g, int R) {
    int RH = (R - 1) * g.stride + g.kh;
    int in_b = RH * tm_row_halves(g) * 2;
    int out_b = (R * g.Q * g.C_out * 2 + 15) / 16 * 16;
    return in_b + out_b;
}

bool tiled_mfma_serves(const ConvGeom& g) {
    return g.K <= 32 && g.C_out <= 32 && tm_lds_bytes(g, 1) <= 64 * 1024;
}

int tiled_mfma_rows(const ConvGeom& g) {
    int R = g.P < 16 ? g.P : 16;
    while (R > 1 && tm_lds_bytes(g, R) > kTmLdsTarget) --R;
    return R;
}

template <int NF, int EPI>
__global__ __launch_bounds__(256) void conv2d_bn_silu_tiled_mfma(
    const f16* __restrict__ x, const f16* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, f16* __restrict__ y, ConvGeom g, int R) {
    extern __shared__ __attribute__((aligned(16))) f16 tm_lds[];
    const int RS = tm_row_halves(g);   // LDS input row (halves)
    const int DO = tm_data_off(g);     // where column 0 starts in a row
    const int bands = (g.P + R - 1) / R;
    const int n = blockIdx.x / bands, band = blockIdx.x - n * bands;
    const int p0 = band * R;
    const int rows_out = imin(R, g.P - p0);
    const int RH = (rows_out - 1) * g.stride + g.kh;
    const int ih0 = p0 * g.stride - g.pad;
    f16* xin = tm_lds;                                  // [RH][RS]
    f16* yout = tm_lds + ((R - 1) * g.stride + g.kh) * RS;  // [rows_out][Q][C_out]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // 1. Input band -> LDS, with zero padding columns and zero rows outside
    //    the image. Rows are contiguous in NHWC: 16-byte copies when aligned.
    const int row_data = g.W * g.C_in;  // halves of one input row
    const bool vec = (row_data & 7) == 0 && (((uintptr_t)x) & 15) == 0;
    // Zeros: the padding columns of every row, and whole rows outside the image.
    const int padh = g.pad * g.C_in, tailh = RS - DO - row_data;
    for (int rr = 0; rr < RH; ++rr) {
        const int ih = ih0 + rr;
        f16* row = xin + rr * RS;
        if ((unsigned)ih >= (unsigned)g.H) {
            for (int e = tid; e < RS; e += 256) row[e] = (f16)0.0f;
        } else {
            if (tid < padh) row[DO - padh + tid] = (f16)0.0f;
            if (tid < tailh) row[DO + row_data + tid] = (f16)0.0f;
        }
    }
    if (!vec) {
        for (int rr = 0; rr < RH; ++rr) {
            const int ih = ih0 + rr;
            if ((unsigned)ih >= (unsigned)g.H) continue;
            const f16* src = x + (size_t)(n * g.H + ih) * row_data;
            for (int e = tid; e < row_data; e += 256) xin[rr * RS + DO + e] = src[e];
        }
    } else {
        const int cpr = row_data / 8;  // 16-byte chunks per row
        for (int i = tid; i < RH * cpr; i += 256) {
            int rr = i / cpr, c = i - rr * cpr;
            int ih = ih0 + rr;
            if ((unsigned)ih < (unsigned)g.H)
                *(half8_t*)(xin + rr * RS + DO + 8 * c) =
                    *(const half8_t*)(x + (size_t)(n * g.H + ih) * row_data + 8 * c);
        }
    }

    // Filter bank in the MFMA row operand: fragment f, lane row lr = channel
    // 16f + lr, k = 8*lg + j (k >= K is zero).
    half8_t wf[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int o = 16 * f + lr;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = 8 * lg + j;
            wf[f][j] = (o < g.C_out && k < g.K) ? w[o * g.K + k] : (f16)0.0f;
        }
    }
    // Gather offsets of this lane's 8 k values within the band (pixel-relative):
    // k = (r*kw + s)*C_in + c -> row r, halves s*C_in + c from the pixel's left edge.
    int koff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int k = 8 * lg + j;
        if (k < g.K) {
            const int L = g.kw * g.C_in;
            const int r = k / L, rem = k - r * L;
            koff[j] = r * RS + rem;
        } else {
            koff[j] = -1;
        }
    }
    float sc[NF][4], bi[NF][4];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            epi_consts<EPI>(scale, bias, 16 * f + 4 * lg + e, g.C_out, sc[f][e], bi[f][e]);
        }
    __syncthreads();

    // 2. 16-pixel runs: (row pl, run j) -> wave w takes runs w, w+4, ...
    const int runs_per_row = (g.Q + 15) / 16;
    const int runs = rows_out * runs_per_row;
    for (int t = wave; t < runs; t += 4) {
        const int pl = t / runs_per_row, q0 = (t - pl * runs_per_row) * 16;
        const int q = q0 + lr;
        const bool qok = q < g.Q;
        const int pbase =
            pl * g.stride * RS + (DO - g.pad * g.C_in) + (qok ? q : 0) * g.stride * g.C_in;
        half8_t b;
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = koff[j] >= 0 ? xin[pbase + koff[j]] : (f16)0.0f;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[f], b, acc, 0, 0, 0);
            const int o = 16 * f + 4 * lg;
            if (qok && o < g.C_out) {
                half4_t h;
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = (f16)epilogue<EPI>(acc[e], sc[f][e], bi[f][e]);
                f16* dst = yout + (pl * g.Q + q) * g.C_out + o;
                if ((g.C_out & 3) == 0) {
                    *(half4_t*)dst = h;  // 8-byte aligned: C_out and o are multiples of 4
                } else {
                    for (int e = 0; e < 4; ++e)
                        if (o + e < g.C_out) dst[e] = h[e];
                }
            }
        }
    }
    __syncthreads();

    // 3. The band's output is one contiguous NHWC range: stream it out.
    const int total = rows_out * g.Q * g.C_out;
    const long long y0 = (long long)(n * g.P + p0) * g.Q * g.C_out;  // first element of y
    const bool vout = ((((uintptr_t)(y + y0)) | ((uintptr_t)yout)) & 15) == 0;
    if (vout) {
        const int nv = total / 8;
        for (int i = tid; i < nv; i += 256)
            store_y8<true>(y, y0 + 8 * i, *(const half8_t*)(yout + 8 * i), g.out8, g.res);
        for (int i = nv * 8 + tid; i < total; i += 256) store_y1(y, y0 + i, yout[i], g.out8, g.res);
    } else {
        for (int i = tid; i < total; i += 256) store_y1(y, y0 + i, yout[i], g.out8, g.res);
    }
}

// Persistent, pipelined form of the same kernel. Requires the band of input
// rows to be one 16-byte aligned contiguous range (W*C_in % 8 == 0) and x
// below 2^31 bytes. Each workgroup walks bands blockIdx.x, +gridDim.x, ...:
// while it computes band i from one LDS buffer, band i+1 streams into the
// other with direct-to-LDS buffer loads (rows above or below the image are
// fetched from neighbouring memory, or past the end as zeros, and masked to
// zero in the gather; padding columns are masked the same way).
template <int NF, int EPI>
__global__ __launch_bounds__(256) void conv2d_bn_silu_tiled_mfma_pipe(
    const f16* __restrict__ x, const f16* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, f16* __restrict__ y, ConvGeom g, int R, int in_halves,
    int nbands_total) {
    extern __shared__ __attribute__((aligned(16))) f16 tm_lds[];
    const int bands = (g.P + R - 1) / R;
    const int row_data = g.W * g.C_in;
    f16* xin[2] = {tm_lds, tm_lds + in_halves};
    f16* yout = tm_lds + 2 * in_halves;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const unsigned xbytes = (unsigned)g.N * g.H * row_data * 2u;
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)xbytes, 0x00020000);
    const int RHmax = (R - 1) * g.stride + g.kh;
    const int chunks = (RHmax * row_data + 511) / 512;  // 1 KB DMA instructions per band

    // Fetch band b's input rows (ih0 .. ih0+RHmax-1, flat) into buffer buf.
    auto fetch = [&](int b, int buf) {
        const int n = b / bands, band = b - n * bands;
        const long long start = ((long long)n * g.H + band * R * g.stride - g.pad) * row_data;
        for (int c = wave; c < chunks; c += 4) {
            const long long e = start + (long long)c * 512 + lane * 8;
            const unsigned off = (e >= 0 && e * 2 < (long long)xbytes) ? (unsigned)(e * 2)
                                                                       : 0x80000000u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (__attribute__((address_space(3))) void*)(xin[buf] + c * 512), 16, off, 0,
                0, 0);
        }
    };

    half8_t wf[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int o = 16 * f + lr;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = 8 * lg + j;
            wf[f][j] = (o < g.C_out && k < g.K) ? w[o * g.K + k] : (f16)0.0f;
        }
    }
    // This lane's 8 k values: filter row kr[j], column kc[j] (within the
    // window) and channel; flat offset within a band koff[j] relative to the
    // window's top-left input element; -1 beyond K.
    int koff[8], kr[8], ks[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int k = 8 * lg + j;
        const int L = g.kw * g.C_in;
        const int r = k / L, rem = k - r * L;
        kr[j] = r;
        ks[j] = rem / g.C_in;
        koff[j] = k < g.K ? r * row_data + rem : -1;
    }
    float sc[NF][4], bi[NF][4];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            epi_consts<EPI>(scale, bias, 16 * f + 4 * lg + e, g.C_out, sc[f][e], bi[f][e]);
        }

    int b = blockIdx.x;
    if (b < nbands_total) fetch(b, 0);
    for (int it = 0; b < nbands_total; b += gridDim.x, ++it) {
        const int buf = it & 1;
        const int nb = b + gridDim.x;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of band b landed
        __syncthreads();  // all of band b in LDS; previous band's output tile fully read
        if (nb < nbands_total) fetch(nb, buf ^ 1);
        const int n = b / bands, band = b - n * bands;
        const int p0 = band * R;
        const int rows_out = imin(R, g.P - p0);
        const int ih0 = p0 * g.stride - g.pad;
        const f16* xb = xin[buf];

        const int runs_per_row = (g.Q + 15) / 16;
        const int runs = rows_out * runs_per_row;
        for (int t = wave; t < runs; t += 4) {
            const int pl = t / runs_per_row, q0 = (t - pl * runs_per_row) * 16;
            const int q = q0 + lr;
            const bool qok = q < g.Q;
            const int iw0 = (qok ? q : 0) * g.stride - g.pad;  // window's left column
            const int rbase = pl * g.stride;                    // window's top row in the band
            const int base = rbase * row_data + iw0 * g.C_in;
            half8_t bv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int ihj = ih0 + rbase + kr[j];
                const int iwj = iw0 + ks[j];
                const bool ok = koff[j] >= 0 && (unsigned)ihj < (unsigned)g.H &&
                                (unsigned)iwj < (unsigned)g.W;
                bv[j] = ok ? xb[base + koff[j]] : (f16)0.0f;
            }
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                float4_t acc = {0.f, 0.f, 0.f, 0.f};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[f], bv, acc, 0, 0, 0);
                const int o = 16 * f + 4 * lg;
                if (qok && o < g.C_out) {
                    half4_t h;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        h[e] = (f16)epilogue<EPI>(acc[e], sc[f][e], bi[f][e]);
                    f16* dst = yout + (pl * g.Q + q) * g.C_out + o;
                    if ((g.C_out & 3) == 0) {
                        *(half4_t*)dst = h;
                    } else {
                        for (int e = 0; e < 4; ++e)
                            if (o + e < g.C_out) dst[e] = h[e];
                    }
                }
            }
        }
        __syncthreads();  // output tile complete
        const int total = rows_out * g.Q * g.C_out;
        const long long y0 = (long long)(n * g.P + p0) * g.Q * g.C_out;  // first element of y
        if (((((uintptr_t)(y + y0)) & 15) == 0) && (total & 7) == 0) {
            for (int i = tid; i < total / 8; i += 256)
                store_y8<true>(y, y0 + 8 * i, *(const half8_t*)(yout + 8 * i), g.out8, g.res);
        } else {
            for (int i = tid; i < total; i += 256) store_y1(y, y0 + i, yout[i], g.out8, g.res);
        }
        // The next iteration's first barrier orders these LDS reads before the
        // next band's writes to the output tile.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}

bool tiled_mfma_pipe_serves(const ConvGeom& g) {
    long long xbytes = 2LL * g.N * g.H * g.W * g.C_in;
    return tiled_mfma_serves(g) && (g.W * g.C_in) % 8 == 0 && xbytes < (1LL << 31) - 4096;
}

int tiled_mfma_pipe_lds(const ConvGeom& g, int R, int* in_halves) {
    int RHmax = (R - 1) * g.stride + g.kh;
    int chunks = (RHmax * g.W * g.C_in + 511) / 512;
    *in_halves = chunks * 512;
    return 2 * chunks * 1024 + (R * g.Q * g.C_out * 2 + 15) / 16 * 16;
}

hipError_t launch_tiled_mfma_pipe(const ConvGeom& g, int R, int grid, int epi,
                                  const void* x, const void* w, const float* scale,
                                  const float* bias, void* y, hipStream_t s) {
    int in_halves = 0;
    const size_t lds = (size_t)tiled_mfma_pipe_lds(g, R, &in_halves);
    const int nbands = g.N * ((g.P + R - 1) / R);
    if (grid > nbands) grid = nbands;
    const int nf = g.C_out <= 16 ? 1 : 2;
#define TG_TMP_LAUNCH(NFV, EPI)                                                              \
    hipLaunchKernelGGL((conv2d_bn_silu_tiled_mfma_pipe<NFV, EPI>), dim3(grid), dim3(256), lds, \
                       s, (const f16*)x, (const f16*)w, scale, bias, (f16*)y, g, R, in_halves, \
                       nbands)
#define TG_TMP_1(E) TG_TMP_LAUNCH(1, E)
#define TG_TMP_2(E) TG_TMP_LAUNCH(2, E)
    if (nf == 1)
        TG_EPI_DISPATCH(epi, TG_TMP_1);
    else
        TG_EPI_DISPATCH(epi, TG_TMP_2);
#undef TG_TMP_2
#undef TG_TMP_1
#undef TG_TMP_LAUNCH
    return hipGetLastError();
}

hipError_t launch_tiled_mfma(const ConvGeom& g, int R, int epi, const void* x,
                             const void* w, const float* scale, const float* bias, void* y,
                             hipStream_t s) {
    const int bands = (g.P + R - 1) / R;
    const size_t lds = (size_t)tm_lds_bytes(g, R);
    dim3 grid(g.N * bands), block(256);
    const int nf = g.C_out <= 16 ? 1 : 2;
#define TG_TM_LAUNCH(NFV, EPI)                                                            \
    hipLaunchKernelGGL((conv2d_bn_silu_tiled_mfma<NFV, EPI>), grid, block, lds, s,         \
                       (const f16*)x, (const f16*)w, scale, bias, (f16*)y, g, R)
#define TG_TM_1(E) TG_TM_LAUNCH(1, E)
#define TG_TM_2(E) TG_TM_LAUNCH(2, E)
    if (nf == 1)
        TG_EPI_DISPATCH(epi, TG_TM_1);
    else
        TG_EPI_DISPATCH(epi, TG_TM_2);
#undef TG_TM_2
#undef TG_TM_1
#undef TG_TM_LAUNCH
    return hipGetLastError();
}

}  // namespace tg
