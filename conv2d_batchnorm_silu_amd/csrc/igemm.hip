// igemm.hip -- conv2d_bn_silu_igemm: the convolution as an implicit GEMM on
// gfx950 fp16 MFMA, with BatchNorm + SiLU applied to the accumulator tile in
// registers before the single store of y.
//
// "Fusing an Epilogue" (teenygrad docs), sections "The shape of it" and "Three
// kernels for one operation": a tiled matmul K-loop leaves the output tile in
// registers; the epilogue scales and shifts it per output channel, applies
// SiLU and only then stores it. Per-channel BatchNorm parameters are loaded
// inside the same kernel; they are tiny next to the tile.
//
// GEMM view (M = N*P*Q output pixels, K = kh*kw*C_in, C_out columns):
//   A[m][k] = x[n][p*stride-pad+r][q*stride-pad+s][c]   (implicit im2col, 0 outside)
//   B[k][o] = w[o][r][s][c]                              (OHWI rows are K-contiguous)
//   with k = (r*kw + s)*C_in + c.
// With C_in % 8 == 0, each aligned run of 8 k values lies inside one filter
// tap, so every operand fetch is one 16-byte load of contiguous NHWC channels.
//
// MFMA mapping (v_mfma_f32_16x16x32_f16, wave64): the instruction's row
// operand is the weight tile (output channels) and its column operand the
// im2col tile (pixels), so each lane's four accumulators hold four
// consecutive output channels of one pixel -- contiguous in NHWC. Lane l reads
// row/column (l % 16) and the 8 consecutive k values 8*(l/16)..+7 of a
// 32-deep step; the accumulator layout (lane l holds column l % 16, rows
// 4*(l/16)+i) was confirmed on gfx950 hardware.
//
// Pipeline: operands for chunk i+1 are fetched from global memory into
// registers while the MFMAs of chunk i read LDS; the registers then go to the
// other LDS buffer; one barrier per chunk. No split-K: the nonlinear epilogue
// needs the complete sum ("Kernel Fusion" cheatsheet, last section: no
// grid-wide barrier exists to finish a split reduction first).
//
// Epilogue: fp32 BN + SiLU per lane, fp16 cast (round to nearest even), the
// tile is transposed through LDS so that each lane stores 16 contiguous bytes
// and a wavefront stores whole NHWC rows.
#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {

template <int BM, int BN, int BK, int WM, int WN>
struct IgemmShape {
    static_assert(WM * WN == 4, "four wavefronts per workgroup");
    static_assert(BK % 32 == 0, "BK is a multiple of the MFMA depth");
    static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile: pixels, channels
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile in 16x16 blocks");
    static constexpr int FM = TM / 16, FN = TN / 16;
    static constexpr int KV = BK / 8;        // 16-byte vectors per row of a chunk
    static constexpr int RPT = 256 / KV;     // rows covered per pass of 256 threads
    static constexpr int XV = (BM + RPT - 1) / RPT;  // x vectors per thread
    static constexpr int WV = (BN + RPT - 1) / RPT;  // w vectors per thread
    static constexpr int LDK = BK + 8;       // padded LDS row (halves): breaks bank aliasing
    static constexpr int STAGE = (BM + BN) * LDK;
    static constexpr int LDO = BN + 8;       // padded row of the output staging tile
    static constexpr int OPER_HALVES = 2 * STAGE;
    static constexpr int OUT_HALVES = BM * LDO;
    static constexpr int SMEM_HALVES = OPER_HALVES > OUT_HALVES ? OPER_HALVES : OUT_HALVES;
};

template <int BM, int BN, int BK, int WM, int WN, int EPI>
__global__ __launch_bounds__(256) void conv2d_bn_silu_igemm(
    const f16* __restrict__ x, const f16* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, f16* __restrict__ y, ConvGeom g, int tiles_m, int tiles_n) {
    using S = IgemmShape<BM, BN, BK, WM, WN>;
    __shared__ __attribute__((aligned(16))) f16 smem[S::SMEM_HALVES];

    const int tile = xcd_contiguous_tile(blockIdx.x, tiles_m * tiles_n);
    const int tm = tile / tiles_n, tn = tile - (tile / tiles_n) * tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave - (wave / WN) * WN;
    const int PQ = g.P * g.Q;

    // Gather state: this thread fetches k-vector `kv` of rows tid/KV + i*RPT.
    const int kv = tid % S::KV;
    const int row0 = tid / S::KV;
    int xbase[S::XV], xh[S::XV], xw[S::XV];
#pragma unroll
    for (int i = 0; i < S::XV; ++i) {
        int row = row0 + i * S::RPT;
        int m = m0 + row;
        if (row < BM && m < g.M) {
            int n = m / PQ, rem = m - n * PQ;
            int p = rem / g.Q, q = rem - p * g.Q;
            xbase[i] = n * g.H * g.W * g.C_in;
            xh[i] = p * g.stride - g.pad;
            xw[i] = q * g.stride - g.pad;
        } else {
            xbase[i] = 0;
            xh[i] = -(1 << 29);  // every ih of this row is out of range
            xw[i] = 0;
        }
    }
    int wbase[S::WV];
    bool wok[S::WV];
#pragma unroll
    for (int i = 0; i < S::WV; ++i) {
        int row = row0 + i * S::RPT;
        int o = n0 + row;
        wok[i] = row < BN && o < g.C_out;
        wbase[i] = wok[i] ? o * g.K : 0;
    }

    half8_t xr[S::XV], wr[S::WV];
    const half8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

    auto gload = [&](int k0) {
        const int k = k0 + kv * 8;
        const bool kok = k < g.K;
        const int tap = k / g.C_in, c = k - tap * g.C_in;
        const int r = tap / g.kw, s = tap - r * g.kw;
#pragma unroll
        for (int i = 0; i < S::XV; ++i) {
            int ih = xh[i] + r, iw = xw[i] + s;
            bool ok = kok && (unsigned)ih < (unsigned)g.H && (unsigned)iw < (unsigned)g.W;
            xr[i] = ok ? *(const half8_t*)(x + xbase[i] + (ih * g.W + iw) * g.C_in + c) : zero8;
        }
#pragma unroll
        for (int i = 0; i < S::WV; ++i)
            wr[i] = (kok && wok[i]) ? *(const half8_t*)(w + wbase[i] + k) : zero8;
    };
    auto sstore = [&](int stage) {
        f16* xs = smem + stage * S::STAGE;
        f16* ws = xs + BM * S::LDK;
#pragma unroll
        for (int i = 0; i < S::XV; ++i) {
            int row = row0 + i * S::RPT;
            if (row < BM) *(half8_t*)(xs + row * S::LDK + kv * 8) = xr[i];
        }
#pragma unroll
        for (int i = 0; i < S::WV; ++i) {
            int row = row0 + i * S::RPT;
            if (row < BN) *(half8_t*)(ws + row * S::LDK + kv * 8) = wr[i];
        }
    };

    float4_t acc[S::FN][S::FM];
#pragma unroll
    for (int a = 0; a < S::FN; ++a)
#pragma unroll
        for (int b = 0; b < S::FM; ++b) acc[a][b] = (float4_t){0.f, 0.f, 0.f, 0.f};

    const int nk = (g.K + BK - 1) / BK;
    const int lrow = lane & 15, lk = (lane >> 4) * 8;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
        const int st = kc & 1;
        if (kc + 1 < nk) gload((kc + 1) * BK);
        const f16* xs = smem + st * S::STAGE;
        const f16* ws = xs + BM * S::LDK;
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            half8_t a[S::FN], b[S::FM];
#pragma unroll
            for (int f = 0; f < S::FN; ++f)
                a[f] = *(const half8_t*)(ws + (wn * S::TN + f * 16 + lrow) * S::LDK + kk + lk);
#pragma unroll
            for (int f = 0; f < S::FM; ++f)
                b[f] = *(const half8_t*)(xs + (wm * S::TM + f * 16 + lrow) * S::LDK + kk + lk);
#pragma unroll
            for (int i = 0; i < S::FN; ++i)
#pragma unroll
                for (int j = 0; j < S::FM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kc + 1 < nk) sstore(st ^ 1);
        __syncthreads();
    }

    // Epilogue in registers: lane holds channels cb..cb+3 of pixel pr per block.
    f16* out = smem;  // operand buffers are free after the last barrier
#pragma unroll
    for (int i = 0; i < S::FN; ++i) {
        const int cb = wn * S::TN + i * 16 + (lane >> 4) * 4;  // channel within tile
        float sc[4], bi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            epi_consts<EPI>(scale, bias, n0 + cb + e, g.C_out, sc[e], bi[e]);
        }
#pragma unroll
        for (int j = 0; j < S::FM; ++j) {
            const int pr = wm * S::TM + j * 16 + lrow;  // pixel within tile
            half4_t h;
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = (f16)epilogue<EPI>(acc[i][j][e], sc[e], bi[e]);
            *(half4_t*)(out + pr * S::LDO + cb) = h;
        }
    }
    __syncthreads();

    // Coalesced store: the tile's rows are NHWC pixel rows of BN channels.
    constexpr int CV = BN / 8;  // 16-byte vectors per tile row
    if ((g.C_out & 7) == 0) {
        for (int v = tid; v < BM * CV; v += 256) {
            int row = v / CV, cv = v - (v / CV) * CV;
            int m = m0 + row, o = n0 + cv * 8;
            if (m < g.M && o < g.C_out)
                store_y8<false>(y, m * g.C_out + o, *(const half8_t*)(out + row * S::LDO + cv * 8), g.out8, g.res);
        }
    } else {
        for (int v = tid; v < BM * BN; v += 256) {
            int row = v / BN, cc = v - (v / BN) * BN;
            int m = m0 + row, o = n0 + cc;
            if (m < g.M && o < g.C_out) store_y1(y, m * g.C_out + o, out[row * S::LDO + cc], g.out8, g.res);
        }
    }
}

// ---- variants ------------------------------------------------------------
#define TG_IGEMM_CFGS(X)      \
    X(128, 128, 32, 2, 2)     \
    X(64, 256, 32, 1, 4)      \
    X(128, 64, 32, 2, 2)      \
    X(208, 64, 32, 1, 4)      \
    X(64, 64, 32, 2, 2)       \
    X(32, 32, 32, 2, 2)

static const IgemmCfg kCfgs[] = {
#define X(bm, bn, bk, wm, wn) {bm, bn, bk, wm, wn},
    TG_IGEMM_CFGS(X)
#undef X
};

int igemm_num_cfgs() { return (int)(sizeof(kCfgs) / sizeof(kCfgs[0])); }
const IgemmCfg& igemm_cfg(int i) { return kCfgs[i]; }

template <int BM, int BN, int BK, int WM, int WN>
static hipError_t launch_one(const ConvGeom& g, int epi, const void* x, const void* w,
                             const float* scale, const float* bias, void* y, hipStream_t s) {
    int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.C_out + BN - 1) / BN;
    dim3 grid(tiles_m * tiles_n), block(256);
#define TG_L(E)                                                                               \
    hipLaunchKernelGGL((conv2d_bn_silu_igemm<BM, BN, BK, WM, WN, E>), grid, block, 0, s,        \
                       (const f16*)x, (const f16*)w, scale, bias, (f16*)y, g, tiles_m, tiles_n)
    TG_EPI_DISPATCH(epi, TG_L);
#undef TG_L
    return hipGetLastError();
}

hipError_t launch_igemm(const ConvGeom& g, int cfg, int epi, const void* x, const void* w,
                        const float* scale, const float* bias, void* y, hipStream_t s) {
    int i = 0;
#define X(bm, bn, bk, wm, wn)                                                                 \
    if (cfg == i) return launch_one<bm, bn, bk, wm, wn>(g, epi, x, w, scale, bias, y, s); \
    ++i;
    TG_IGEMM_CFGS(X)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace tg
