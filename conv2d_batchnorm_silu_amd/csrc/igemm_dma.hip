// igemm_dma.hip -- conv2d_bn_silu_igemm for long reductions (MFMA-bound
// layers such as 3x3 and 7x7 convolutions with 64+ input channels).
//
// The operation is that of igemm.hip ("Fusing an Epilogue", teenygrad docs,
// "The shape of it": a tiled K-loop on the matrix cores, then the per-channel
// BatchNorm scale/shift and SiLU on the register tile, then one store). This
// variant is built for gfx950 throughput when C_in % 64 == 0:
//   * A K-chunk is 64 input channels of one filter tap, so every pixel's
//     chunk (and every filter row's chunk) is one aligned 128-byte line.
//   * Operands go global -> LDS with direct-to-LDS buffer loads: each load
//     instruction moves 8 full lines (1 KB) and costs no VGPRs. Taps outside
//     the image get an out-of-range offset and read as zeros.
//   * The loads scatter each line's eight 16-byte pieces over an XOR-swizzled
//     slot order (slot = piece ^ (row16 >> 1)), which makes the MFMA fragment
//     reads (16 rows x one 16-byte piece) bank-conflict-free.
//   * A RING-stage ring keeps RING-1 chunks in flight; one workgroup barrier
//     per chunk. The main loop issues no stores, so waiting for the oldest
//     chunk's loads is an exact vmcnt wait.
//   * WK = 2 runs two groups of four waves, each taking one 32-deep half of
//     every chunk, so each SIMD holds two waves and one wave's fragment reads
//     overlap the other's MFMAs (with one wave per SIMD the two alternate).
//     The two partial tiles are summed through LDS before the epilogue; the
//     sum is over the complete K, as the nonlinear epilogue requires.
//   * Epilogue: fp32 BatchNorm + SiLU on the accumulators, fp16 cast, then
//     the tile goes through LDS so each store instruction writes whole
//     128-byte lines of NHWC rows.
// No split-K: the nonlinear epilogue needs the complete sum.
#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {

__device__ __forceinline__ void dma_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void dma_wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// BM pixels x BN channels per workgroup of 4*WK waves: WK groups of 4 waves
// arranged WM x WN; FM x FN 16x16 blocks per wave; RING LDS stages of one
// 64-deep chunk.
template <int BM, int BN, int WM, int WN, int RING, int WK>
struct DmaShape {
    static_assert(WM * WN == 4, "four waves per K-group");
    static_assert(WK == 1 || WK == 2, "one or two K-groups");
    static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tiles of 16x16 blocks");
    static_assert(BM % 16 == 0 && BN % 16 == 0, "16-row swizzle groups");
    static constexpr int NW = 4 * WK;                // waves per workgroup
    static constexpr int FM = BM / WM / 16, FN = BN / WN / 16;
    static constexpr int XI = BM / 8, WI = BN / 8;   // load instructions per chunk
    static constexpr int LI = (XI + WI + NW - 1) / NW;  // per wave (padded with repeats)
    static constexpr int STAGE = (BM + BN) * 64;     // halves per stage
    static constexpr int OROW = BN + 8;              // output tile row (halves)
    // K-group 1's partial accumulators (fp32, lane-major per 16x16 block),
    // then the output tile; both overlay the ring after the main loop.
    static constexpr int RED = WK == 2 ? 4 * FN * FM * 64 * 4 * 2 : 0;  // halves
    static constexpr int OUT_AT = RED;
    static constexpr int EPI_SMEM = RED + BM * OROW;
    static constexpr int SMEM = RING * STAGE > EPI_SMEM ? RING * STAGE : EPI_SMEM;
    static_assert(LI * (RING - 1) <= 63, "vmcnt range");
};

template <int BM, int BN, int WM, int WN, int RING, int WK, int EPI>
__global__ __launch_bounds__(256 * WK, 1) void conv2d_bn_silu_igemm_dma(
    const f16* __restrict__ x, const f16* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, f16* __restrict__ y, ConvGeom g, int tiles_m, int tiles_n) {
    using S = DmaShape<BM, BN, WM, WN, RING, WK>;
    extern __shared__ __attribute__((aligned(16))) f16 dma_smem[];

    const int tile = xcd_contiguous_tile(blockIdx.x, tiles_m * tiles_n);
    const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    // Wave-uniform by construction; readfirstlane lets the compiler keep the
    // load-assignment choices below (buffer and LDS destination) scalar.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = wave >> 2, w4 = wave & 3;  // K-group, wave within it
    const int wm = w4 / WN, wn = w4 - (w4 / WN) * WN;
    const int lr = lane & 15, lg = lane >> 4;
    const int PQ = g.P * g.Q;
    const int cchunks = g.C_in / 64;          // chunks per filter tap
    const int nk = g.kh * g.kw * cchunks;     // chunks in K

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)x, (short)0, (int)((unsigned)g.N * g.H * g.W * g.C_in * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)w, (short)0, (int)((unsigned)g.C_out * g.K * 2u), 0x00020000);
    const unsigned kOut = 0x80000000u;  // beyond both buffers (each is below 2^31 bytes)

    // Load assignment: instruction j (of XI x-instructions then WI
    // w-instructions) covers rows 8*(j')..8*(j')+7; lane l takes row
    // 8*j' + l/8 and piece (l%8) ^ ((row % 16) >> 1), written to slot l%8.
    // Each wave issues LI instructions j = wave + NW*i (clamped: repeats of
    // the last instruction write identical data to the same place).
    const int prow = lane >> 3, pslot = lane & 7;
    int base_x[S::LI], h0[S::LI], w0[S::LI], piece[S::LI];
    bool kind[S::LI];   // wave-uniform: x (true) or w (false) instruction
    int srow0[S::LI];   // wave-uniform: first stage row of the instruction
#pragma unroll
    for (int i = 0; i < S::LI; ++i) {
        int j = wave + S::NW * i;
        if (j > S::XI + S::WI - 1) j = S::XI + S::WI - 1;
        const bool isx = j < S::XI;
        const int row0 = (isx ? j : j - S::XI) * 8;         // first tile row (uniform)
        const int row = row0 + prow;                        // this lane's row
        kind[i] = isx;
        srow0[i] = isx ? row0 : BM + row0;
        piece[i] = pslot ^ ((row & 15) >> 1);
        if (isx) {
            const int m = m0 + row;
            if (m < g.M) {
                int n = m / PQ, rem = m - n * PQ;
                int p = rem / g.Q, q = rem - p * g.Q;
                base_x[i] = n * g.H * g.W;
                h0[i] = p * g.stride - g.pad;
                w0[i] = q * g.stride - g.pad;
            } else {
                base_x[i] = 0;
                h0[i] = -(1 << 29);
                w0[i] = 0;
            }
        } else {
            const int o = n0 + row;
            base_x[i] = o < g.C_out ? o : -1;  // filter row, or -1 beyond C_out
            h0[i] = 0;
            w0[i] = 0;
        }
    }
    // Issue chunk kc (tap r,s; channels c0..c0+63) into stage kc % RING.
    auto issue = [&](int kc) {
        const int tap = kc / cchunks, c0 = (kc - tap * cchunks) * 64;
        const int r = tap / g.kw, s = tap - r * g.kw;
        f16* st = dma_smem + (kc % RING) * S::STAGE;
#pragma unroll
        for (int i = 0; i < S::LI; ++i) {
            f16* dst = st + srow0[i] * 64;  // 8 rows of 64 halves = 1 KB, lane-major
            if (kind[i]) {
                const int ih = h0[i] + r, iw = w0[i] + s;
                const bool ok = (unsigned)ih < (unsigned)g.H && (unsigned)iw < (unsigned)g.W;
                const unsigned off =
                    ok ? (unsigned)(((base_x[i] + ih * g.W + iw) * g.C_in + c0 + piece[i] * 8) * 2)
                       : kOut;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xr, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
            } else {
                const unsigned off =
                    base_x[i] >= 0
                        ? (unsigned)((base_x[i] * g.K + tap * g.C_in + c0 + piece[i] * 8) * 2)
                        : kOut;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    wr, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
            }
        }
    };

    float4_t acc[S::FN][S::FM];
#pragma unroll
    for (int a = 0; a < S::FN; ++a)
#pragma unroll
        for (int b = 0; b < S::FM; ++b) acc[a][b] = (float4_t){0.f, 0.f, 0.f, 0.f};

    // Prologue: RING-1 chunks in flight.
    int issued = 0;
    for (; issued < RING - 1 && issued < nk; ++issued) issue(issued);

    for (int kc = 0; kc < nk; ++kc) {
        // This wave's loads for chunk kc are done when at most (issued-kc-1)
        // later chunks' loads are pending.
        switch (issued - kc - 1) {
            case 0: dma_wait_vmcnt<0>(); break;
            case 1: dma_wait_vmcnt<S::LI>(); break;
            case 2: if (RING > 3) dma_wait_vmcnt<(RING > 3 ? 2 * S::LI : 0)>(); break;
            default: if (RING > 4) dma_wait_vmcnt<(RING > 4 ? 3 * S::LI : 0)>(); break;
        }
        dma_barrier();  // chunk kc visible to all; stage of chunk kc-1 free
        if (issued < nk) issue(issued++);
        const f16* st = dma_smem + (kc % RING) * S::STAGE;
#pragma unroll
        for (int kk = 0; kk < 2 / WK; ++kk) {
            const int ks = WK == 2 ? kg : kk;  // 32-deep half of the chunk
            const int pc = ks * 4 + lg;  // 16-byte piece of the 128-byte chunk row
            half8_t a[S::FN], b[S::FM];
#pragma unroll
            for (int f = 0; f < S::FN; ++f) {
                const int row = wn * S::FN * 16 + f * 16 + lr;
                a[f] = *(const half8_t*)(st + (BM + row) * 64 + ((pc ^ (lr >> 1)) * 8));
            }
#pragma unroll
            for (int f = 0; f < S::FM; ++f) {
                const int row = wm * S::FM * 16 + f * 16 + lr;
                b[f] = *(const half8_t*)(st + row * 64 + ((pc ^ (lr >> 1)) * 8));
            }
#pragma unroll
            for (int i = 0; i < S::FN; ++i)
#pragma unroll
                for (int j = 0; j < S::FM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }
    dma_barrier();  // all waves done with the ring: reuse it for the output tile

    if (WK == 2) {
        // Sum the two K-groups' partial tiles: group 1 parks its accumulators
        // in LDS (each lane 16 contiguous bytes per block), group 0 adds them.
        float4_t* red = (float4_t*)dma_smem + w4 * S::FN * S::FM * 64 + lane;
        if (kg == 1) {
#pragma unroll
            for (int i = 0; i < S::FN; ++i)
#pragma unroll
                for (int j = 0; j < S::FM; ++j) red[(i * S::FM + j) * 64] = acc[i][j];
        }
        dma_barrier();
        if (kg == 1) goto store_phase;
#pragma unroll
        for (int i = 0; i < S::FN; ++i)
#pragma unroll
            for (int j = 0; j < S::FM; ++j) acc[i][j] += red[(i * S::FM + j) * 64];
    }

    {
    // Epilogue: lane holds channels cb..cb+3 of pixel pr for each block.
    f16* out = dma_smem + S::OUT_AT;
#pragma unroll
    for (int i = 0; i < S::FN; ++i) {
        const int cb = wn * S::FN * 16 + i * 16 + lg * 4;
        float sc[4], bi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            epi_consts<EPI>(scale, bias, n0 + cb + e, g.C_out, sc[e], bi[e]);
        }
#pragma unroll
        for (int j = 0; j < S::FM; ++j) {
            const int pr = wm * S::FM * 16 + j * 16 + lr;
            half4_t h;
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = (f16)epilogue<EPI>(acc[i][j][e], sc[e], bi[e]);
            *(half4_t*)(out + pr * S::OROW + cb) = h;
        }
    }
    }

store_phase:
    dma_barrier();
    {
    const f16* out = dma_smem + S::OUT_AT;
    constexpr int CV = BN / 8;  // 16-byte pieces per tile row
    if ((g.C_out & 7) == 0) {
        for (int v = threadIdx.x; v < BM * CV; v += 64 * S::NW) {
            const int row = v / CV, cv = v - (v / CV) * CV;
            const int m = m0 + row, o = n0 + cv * 8;
            if (m < g.M && o < g.C_out)
                store_y8<false>(y, m * g.C_out + o, *(const half8_t*)(out + row * S::OROW + cv * 8), g.out8, g.res);
        }
    } else {
        for (int v = threadIdx.x; v < BM * BN; v += 64 * S::NW) {
            const int row = v / BN, cc = v - (v / BN) * BN;
            const int m = m0 + row, o = n0 + cc;
            if (m < g.M && o < g.C_out) store_y1(y, m * g.C_out + o, out[row * S::OROW + cc], g.out8, g.res);
        }
    }
    }
}

// ---- variants ------------------------------------------------------------
#define TG_DMA_CFGS(X)           \
    X(128, 128, 2, 2, 4, 1)      \
    X(112, 128, 1, 4, 4, 1)      \
    X(208, 64, 1, 4, 4, 1)       \
    X(224, 64, 2, 2, 4, 1)       \
    X(128, 64, 2, 2, 4, 1)       \
    X(64, 64, 2, 2, 4, 1)        \
    X(128, 128, 2, 2, 4, 2)      \
    X(112, 128, 1, 4, 4, 2)      \
    X(208, 64, 1, 4, 4, 2)       \
    X(224, 64, 2, 2, 4, 2)       \
    X(128, 64, 2, 2, 4, 2)

static const IgemmCfg kDmaCfgs[] = {
#define X(bm, bn, wm, wn, ring, wk) {bm, bn, 64, wm, wn, wk},
    TG_DMA_CFGS(X)
#undef X
};

int igemm_dma_num_cfgs() { return (int)(sizeof(kDmaCfgs) / sizeof(kDmaCfgs[0])); }
const IgemmCfg& igemm_dma_cfg(int i) { return kDmaCfgs[i]; }

bool igemm_dma_serves(const ConvGeom& g) {
    long long xbytes = 2LL * g.N * g.H * g.W * g.C_in, wbytes = 2LL * g.C_out * g.K;
    return g.C_in % 64 == 0 && xbytes < (1LL << 31) && wbytes < (1LL << 31);
}

template <int BM, int BN, int WM, int WN, int RING, int WK>
static hipError_t dma_launch_one(const ConvGeom& g, int epi, const void* x, const void* w,
                                 const float* scale, const float* bias, void* y, hipStream_t s) {
    using S = DmaShape<BM, BN, WM, WN, RING, WK>;
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.C_out + BN - 1) / BN;
    const size_t lds = (size_t)S::SMEM * 2;
    static_assert(S::SMEM * 2 <= 160 * 1024, "LDS budget");
    if (epi < 0 || epi >= kNumEpilogues) return hipErrorInvalidValue;
    auto k = conv2d_bn_silu_igemm_dma<BM, BN, WM, WN, RING, WK, EPI_FUSED>;
#define TG_K(E) k = conv2d_bn_silu_igemm_dma<BM, BN, WM, WN, RING, WK, E>
    TG_EPI_DISPATCH(epi, TG_K);
#undef TG_K
    hipError_t e = ensure_dynamic_lds((const void*)k, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(tiles_m * tiles_n), dim3(64 * S::NW), lds, s, (const f16*)x,
                       (const f16*)w,
                       scale, bias, (f16*)y, g, tiles_m, tiles_n);
    return hipGetLastError();
}

hipError_t launch_igemm_dma(const ConvGeom& g, int cfg, int epi, const void* x,
                            const void* w, const float* scale, const float* bias, void* y,
                            hipStream_t s) {
    int i = 0;
#define X(bm, bn, wm, wn, ring, wk)                                                         \
    if (cfg == i) return dma_launch_one<bm, bn, wm, wn, ring, wk>(g, epi, x, w, scale,      \
                                                                  bias, y, s);              \
    ++i;
    TG_DMA_CFGS(X)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace tg
