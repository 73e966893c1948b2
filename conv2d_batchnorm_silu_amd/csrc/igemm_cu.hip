// igemm_cu.hip -- conv2d_bn_silu_igemm for the 1x1 channel-mixing layer with
// 64 input channels (K = 64) and C_out a multiple of 64 up to 256: one
// persistent workgroup per compute unit.
//
// The operation is the same as in igemm.hip ("Fusing an Epilogue", teenygrad
// docs, "The shape of it": the K-loop leaves the output tile in registers,
// BatchNorm scale/shift and SiLU are applied there, then one store). This
// shape is a store stream (about 51 FLOP per byte of HBM traffic, 4 bytes of
// y written per byte of x read), so the design is about keeping HBM busy from
// the first to the last cycle of the launch:
//   * One workgroup per compute unit (its LDS request exceeds half of the
//     160 KB, so the dispatcher cannot stack two on one unit while another
//     idles). It owns one contiguous range of 16-pixel blocks.
//   * The filter bank (C_out x 64 fp16) and the folded BatchNorm constants
//     are fetched once per workgroup with direct-to-LDS loads, in parallel
//     with the first input blocks, instead of once per wavefront from L2.
//     Filter rows are stored with an XOR swizzle so that the fragment reads
//     are free of bank conflicts.
//   * Each wavefront owns one 64-channel slice (weights in VGPRs, rows
//     permuted so that a lane's accumulators hold 8 consecutive channels of
//     one pixel) and pulls blocks of the workgroup's range from a per-slice
//     LDS counter, so fast and slow SIMDs finish together.
//   * Input blocks (16 pixels x 128 bytes, one full line per pixel) are
//     prefetched PD blocks ahead straight into LDS. Vector loads and stores
//     share one completion counter, so the wait for a prefetched block is an
//     exact count that leaves the stores issued after it in flight.
//   * Results go through a small wave-private LDS tile so that each store
//     instruction writes whole 128-byte pieces of 8 pixel rows.
//   * Training mode (STATS): the kernel accumulates the per-channel batch
//     statistics from the fp32 accumulators ("Kernel Fusion", cheatsheet
//     page: a reduction next to elementwise work takes one or two passes)
//     and stores nothing; the training call then runs the fused kernel with
//     the folded batch statistics, which computes the conv again (the layer
//     is bound by HBM, and reading x twice costs less than writing t1 and
//     reading and writing it again). Each lane sums
//     d = acc - shift and d^2 over its pixels, with one shift per channel
//     shared by the 16 lanes of a row (a value of the channel, so that the
//     sum of squares does not cancel when the mean is far from 0); the
//     row's sums become a (count, mean, sum of squared deviations) triple in
//     fp64, and the waves of a slice combine theirs with the pairwise update
//     of Chan, Golub and LeVeque (1979), all in a fixed order. Blocks are
//     then assigned round-robin instead of pulled from the counter, so the
//     result does not depend on scheduling.
#include <stdlib.h>

#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {
namespace {

constexpr int kCuMinLdsBytes = 81 * 1024;   // more than half of a CU's LDS
constexpr int kCuMaxLdsBytes = 160 * 1024 - 64;  // 160 KB minus the static counters
constexpr int kCuCW = 64;                  // channels per wavefront slice
constexpr int kCuTrow = kCuCW + 8;         // padded tile row (halves)
constexpr int kCuStatsThreads = 768;       // at most 12 waves with the statistics registers

template <int N>
__device__ __forceinline__ void cu_wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte direct-to-LDS buffer load: lane l's bytes land at lds + 16*l;
// offsets at or past num_records read as zeros. Inline assembly, so the
// compiler adds no wait of its own for the LDS write: callers order it with
// explicit vmcnt waits and a barrier. lds must be wave-uniform.
__device__ __forceinline__ void cu_dma16(u32x4_t rsrc, unsigned voff, unsigned lds) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds)
                 : "memory");
}

__device__ __forceinline__ u32x4_t cu_rsrc(const void* base, unsigned bytes) {
    const unsigned long long a = (unsigned long long)base;
    u32x4_t r;
    r[0] = (unsigned)a;
    r[1] = (unsigned)(a >> 32) & 0xffffu;  // stride 0
    r[2] = bytes;                          // num_records: reads past it return 0
    r[3] = 0x00020000u;
    return r;
}

// Keeps the compiler from moving one wave's LDS accesses across this point;
// the LDS itself executes a wave's operations in order.
__device__ __forceinline__ void cu_wave_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// Output channel of row i of weight fragment f within a 64-channel slice.
__device__ __forceinline__ int cu_sigma(int f, int i) {
    return 32 * (f >> 1) + 8 * (i >> 2) + 4 * (f & 1) + (i & 3);
}

// Filter row r's 16-byte piece p lives in slot p ^ cu_wswz(r) of the row. The
// 8 lanes of one LDS pass read rows base + {0..3, 8..11} at one piece; this
// maps them to 8 distinct slots.
__device__ __forceinline__ int cu_wswz(int r) { return (r & 3) | ((r >> 1) & 4); }

struct CuLayout {
    int w_off, s_off, b_off, x_off, t_off, bytes;
};

__host__ __device__ inline CuLayout cu_layout(int C_out, int nwaves, int pd) {
    CuLayout L;
    L.w_off = 0;
    L.s_off = C_out * 128;
    L.b_off = L.s_off + 1024;
    L.x_off = L.b_off + 1024;
    L.t_off = L.x_off + nwaves * pd * 2048;
    L.bytes = L.t_off + nwaves * 16 * kCuTrow * 2;
    return L;
}

// STATS: the per-workgroup statistics into stats and nothing stored to y.
template <int EPI, bool NT, int PD, bool OUT8, bool RES, bool STATS>
__global__ __launch_bounds__(STATS ? kCuStatsThreads : 1024) void conv2d_bn_silu_igemm_cu(
    const f16* __restrict__ x, const f16* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, f16* __restrict__ y, int M, int C_out, int nwaves,
    const f16* __restrict__ res, double* __restrict__ stats) {
    constexpr int NF = 4, KS = 2;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ int next_blk[4];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int ngroups = C_out / kCuCW;
    const int grp = wave % ngroups, rnk = wave / ngroups, R = nwaves / ngroups;
    const int c0 = grp * kCuCW;
    const int nblocks = (M + 15) / 16;
    const int b_begin = (int)((long long)blockIdx.x * nblocks / gridDim.x);
    const int b_end = (int)((long long)(blockIdx.x + 1) * nblocks / gridDim.x);
    const CuLayout L = cu_layout(C_out, nwaves, PD);
    const unsigned lbase =
        (unsigned)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)lds);

    if (threadIdx.x < 4) next_blk[threadIdx.x] = b_begin + R * PD;

    // Filter bank: C_out rows of 128 bytes, 8 rows per instruction.
    const u32x4_t wrs = cu_rsrc(w, (unsigned)C_out * 128u);
    for (int h = wave; h < C_out / 8; h += nwaves) {
        const int row = 8 * h + (lane >> 3);
        const int piece = (lane & 7) ^ cu_wswz(row);
        cu_dma16(wrs, (unsigned)(row * 128 + piece * 16), lbase + L.w_off + h * 1024);
    }
    // Scale and bias: up to 256 floats each, one instruction each (none for
    // the identity epilogue, which does not read them; they may be NULL).
    if (EPI != EPI_IDENTITY && wave == 0)
        cu_dma16(cu_rsrc(scale, (unsigned)C_out * 4u), lane * 16u, lbase + L.s_off);
    if (EPI != EPI_IDENTITY && wave == (nwaves > 1 ? 1 : 0))
        cu_dma16(cu_rsrc(bias, (unsigned)C_out * 4u), lane * 16u, lbase + L.b_off);

    // Input block b: pixels 16b..16b+15, 128 bytes each. Instruction h moves
    // pixels 8h..8h+7: lane l -> pixel 8h + l/8, slot l%8 holds piece
    // (l%8) ^ ((pixel >> 1) & 7), which makes the fragment reads conflict-free.
    const unsigned xbytes = (unsigned)M * 128u;
    const u32x4_t xrs = cu_rsrc(x, xbytes);
    const unsigned xbuf0 = lbase + L.x_off + (unsigned)wave * PD * 2048u;
    auto fetch = [&](int blk, int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int px = 8 * h + (lane >> 3);
            const int piece = (lane & 7) ^ ((px >> 1) & 7);
            const int m = blk * 16 + px;
            const unsigned off =
                (blk < b_end && m < M) ? (unsigned)(m * 128 + piece * 16) : 0x80000000u;
            cu_dma16(xrs, off, xbuf0 + (unsigned)buf * 2048u + h * 1024u);
        }
    };
    int q[PD];  // blocks whose input is in flight, oldest first
#pragma unroll
    for (int d = 0; d < PD; ++d) {
        q[d] = b_begin + rnk + R * d;
        fetch(q[d], d);
    }
    // Everything but the 2*PD input loads just issued has landed, for every
    // wave once the barrier is passed.
    cu_wait_vmcnt<2 * PD>();
    __syncthreads();

    half8_t wf[NF][KS];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int row = c0 + cu_sigma(f, lr), piece = 4 * s + lg;
            wf[f][s] = *(const half8_t*)(lds + L.w_off + row * 128 + (piece ^ cu_wswz(row)) * 16);
        }
    // Lane (lr, lg) owns channels c0 + 32*j + 8*lg + [0, 8) for j < 2.
    float sc[NF / 2][8], bi[NF / 2][8];
#pragma unroll
    for (int j = 0; j < NF / 2; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int o = c0 + 32 * j + 8 * lg + e;
            sc[j][e] = epi_scale<EPI>(((const float*)(lds + L.s_off))[o]);
            bi[j][e] = epi_scale<EPI>(((const float*)(lds + L.b_off))[o]);
        }

    f16* tl = (f16*)(lds + L.t_off) + wave * 16 * kCuTrow;
    const int ocs = (lane % 8) * 8;  // channel within the slice, store phase
    const int orow = lane / 8;       // first tile row, store phase
    // Element offsets in y of this lane's two stores, less the block's
    // (every element index of y fits 31 bits, checked at plan creation).
    const int soff0 = orow * C_out + c0 + ocs, soff1 = soff0 + 8 * C_out;
    // Statistics: lane (lr, lg) sees pixel lr of each of its blocks and
    // channels c0 + 32*(f/2) + 8*lg + 4*(f%2) + e of accumulator f, element e.
    float st_shift[NF][4], st_s1[NF][4], st_s2[NF][4];
    int st_n = 0;
    if (STATS) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int e = 0; e < 4; ++e) st_shift[f][e] = st_s1[f][e] = st_s2[f][e] = 0.0f;
    }
    for (int it = 0;; ++it) {
        const int blk = q[0];
        if (blk >= b_end) break;
        int nb = 0;
        if (STATS) {
            nb = q[PD - 1] + R;  // round-robin: rank rnk takes b_begin + rnk + R*i
        } else {
            if (lane == 0) nb = atomicAdd(&next_blk[grp], 1);
            nb = __builtin_amdgcn_readfirstlane(nb);
        }
        // Exact wait for block blk's two loads. Each iteration issues two
        // loads (after its MFMAs) and two stores, so they are followed by
        // 2*(PD-1-it) + 4*it operations while it < PD and 4*PD-2 afterwards.
        // Without stores (STATS) only the other PD - 1 blocks' loads follow.
        if (STATS || it < PD) cu_wait_vmcnt<2 * (PD - 1)>(); else cu_wait_vmcnt<4 * PD - 2>();
        const int buf = it % PD;
        const f16* xb = (const f16*)(lds + L.x_off) + (wave * PD + buf) * 1024;
        half8_t xc[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int pc = 4 * s + lg;
            xc[s] = *(const half8_t*)(xb + lr * 64 + ((pc ^ (lr >> 1)) & 7) * 8);
        }
        float4_t acc[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[f] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int f = 0; f < NF; ++f)
                acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[f][s], xc[s], acc[f], 0, 0, 0);
        if (STATS) {
            // One shift per channel for the 16 lanes of a row: the value of
            // the row's lane 0 in the first block (pixel 0 of a block is
            // always inside the image), so the lanes' sums add directly.
            // Pixels past M add nothing.
            if (it == 0) {
#pragma unroll
                for (int f = 0; f < NF; ++f)
#pragma unroll
                    for (int e = 0; e < 4; ++e) st_shift[f][e] = __shfl(acc[f][e], lane & 48);
            }
            if (blk * 16 + 16 <= M) {  // whole block (wave-uniform)
                ++st_n;
#pragma unroll
                for (int f = 0; f < NF; ++f)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float d = acc[f][e] - st_shift[f][e];
                        st_s1[f][e] += d;
                        st_s2[f][e] = __builtin_fmaf(d, d, st_s2[f][e]);
                    }
            } else {  // the last block of the image batch
                const bool valid = blk * 16 + lr < M;
                st_n += valid ? 1 : 0;
#pragma unroll
                for (int f = 0; f < NF; ++f)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float d = valid ? acc[f][e] - st_shift[f][e] : 0.0f;
                        st_s1[f][e] += d;
                        st_s2[f][e] = __builtin_fmaf(d, d, st_s2[f][e]);
                    }
            }
        }
        fetch(nb, buf);  // the fragment reads above have completed (the MFMAs used them)
#pragma unroll
        for (int d = 0; d + 1 < PD; ++d) q[d] = q[d + 1];
        q[PD - 1] = nb;
        if constexpr (STATS) continue;
#pragma unroll
        for (int j = 0; j < NF / 2; ++j) {
            half8_t h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h[e] = (f16)epilogue<EPI>(acc[2 * j][e], sc[j][e], bi[j][e]);
                h[4 + e] = (f16)epilogue<EPI>(acc[2 * j + 1][e], sc[j][4 + e], bi[j][4 + e]);
            }
            *(half8_t*)(tl + lr * kCuTrow + 32 * j + 8 * lg) = h;
        }
        cu_wave_sync();
        const int yb = blk * 16 * C_out;  // the block's first element of y
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = orow + 8 * i;
            const int m = blk * 16 + row;
            const half8_t v = *(const half8_t*)(tl + row * kCuTrow + ocs);
            if (m < M)
                store_y8<NT>(y, (long long)(unsigned)(yb + (i == 0 ? soff0 : soff1)), v,
                             OUT8 ? 1 : 0, RES ? (const void*)res : nullptr);
        }
        cu_wave_sync();
    }
    if constexpr (STATS) {
        // The 16 lanes of a row share their shifts: add their counts and
        // sums across the row (every lane ends with the row's totals), then
        // form the row's (count, mean, squared deviations) in fp64.
        const float nrow = row_sum16((float)st_n);  // at most 16 x blocks: exact
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                st_s1[f][e] = row_sum16(st_s1[f][e]);
                st_s2[f][e] = row_sum16(st_s2[f][e]);
            }
        double sn[NF][4], smean[NF][4], sm2[NF][4];
        const double n0 = (double)nrow;
        const double inv_n = nrow > 0.0f ? 1.0 / n0 : 0.0;
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double s1 = st_s1[f][e], s2 = st_s2[f][e];
                sn[f][e] = n0;
                smean[f][e] = nrow > 0.0f ? (double)st_shift[f][e] + s1 * inv_n : 0.0;
                const double m2 = s2 - s1 * s1 * inv_n;
                sm2[f][e] = m2 > 0.0 ? m2 : 0.0;
            }
        // The wave's triples (64 channels) go to its own input-buffer space
        // once its last (zero-filled) prefetches have landed; then rank 0 of
        // each slice merges the ranks in order and writes the workgroup's
        // triples: stats[(blockIdx.x * C_out + c) * 3 + {0, 1, 2}].
        cu_wait_vmcnt<0>();
        double* wt = (double*)(lds + L.x_off + (unsigned)wave * PD * 2048u);
        if (lr == 0) {
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int cl = 32 * (f >> 1) + 8 * lg + 4 * (f & 1) + e;
                    wt[cl * 3 + 0] = sn[f][e];
                    wt[cl * 3 + 1] = smean[f][e];
                    wt[cl * 3 + 2] = sm2[f][e];
                }
        }
        __syncthreads();
        if (rnk == 0) {
            double n = 0.0, mean = 0.0, m2 = 0.0;
            for (int r = 0; r < R; ++r) {
                const double* src =
                    (const double*)(lds + L.x_off + (unsigned)(grp + r * ngroups) * PD * 2048u);
                chan_merge(n, mean, m2, src[lane * 3], src[lane * 3 + 1], src[lane * 3 + 2]);
            }
            double* dst = stats + ((size_t)blockIdx.x * C_out + c0 + lane) * 3;
            dst[0] = n;
            dst[1] = mean;
            dst[2] = m2;
        }
    }
}

template <int EPI, bool NT, int PD, bool OUT8, bool RES, bool STATS = false>
hipError_t launch_cu_t(const ConvGeom& g, int grid, int nwaves, const void* x, const void* w,
                       const float* scale, const float* bias, void* y, hipStream_t s,
                       double* stats = nullptr) {
    const CuLayout L = cu_layout(g.C_out, nwaves, PD);
    if (L.bytes > kCuMaxLdsBytes) return hipErrorInvalidValue;
    const int lds = L.bytes > kCuMinLdsBytes ? L.bytes : kCuMinLdsBytes;
    hipError_t e = ensure_dynamic_lds(
        (const void*)conv2d_bn_silu_igemm_cu<EPI, NT, PD, OUT8, RES, STATS>, (size_t)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((conv2d_bn_silu_igemm_cu<EPI, NT, PD, OUT8, RES, STATS>), dim3(grid),
                       dim3(64 * nwaves), lds, s, (const f16*)x, (const f16*)w, scale, bias,
                       (f16*)y, g.M, g.C_out, nwaves, (const f16*)g.res, stats);
    return hipGetLastError();
}

}  // namespace

bool igemm_cu_serves(const ConvGeom& g) {
    return g.kh == 1 && g.kw == 1 && g.stride == 1 && g.pad == 0 && g.C_in == 64 &&
           g.C_out % kCuCW == 0 && g.C_out <= 256 && (long long)g.M * 128 < (1LL << 31);
}

int igemm_cu_waves(const ConvGeom& g, int per_group) {
    int ng = g.C_out / kCuCW;
    int r = per_group < 1 ? 1 : per_group;
    while (ng * r > 16) --r;
    return ng * r;
}

hipError_t launch_igemm_cu(const ConvGeom& g, int nwaves, int pd, bool nt, int epi,
                           const void* x, const void* w, const float* scale, const float* bias,
                           void* y, hipStream_t s) {
    if (!igemm_cu_serves(g) || nwaves < 1 || nwaves > 16 || nwaves % (g.C_out / kCuCW) != 0)
        return hipErrorInvalidValue;
    const int nblocks = (g.M + 15) / 16;
    const int grid = nblocks < 256 ? nblocks : 256;
    if (grid == 0) return hipSuccess;
#define TG_CU(EPI, NTV, PDV) \
    return g.out8  ? launch_cu_t<EPI, NTV, PDV, true, false>(g, grid, nwaves, x, w, scale, bias, y, s) \
           : g.res ? launch_cu_t<EPI, NTV, PDV, false, true>(g, grid, nwaves, x, w, scale, bias, y, s) \
                   : launch_cu_t<EPI, NTV, PDV, false, false>(g, grid, nwaves, x, w, scale, bias, y, s)
#define TG_CU_PD(EPI, NTV)              \
    do {                                \
        if (pd <= 1) TG_CU(EPI, NTV, 1); \
        if (pd == 2) TG_CU(EPI, NTV, 2); \
        TG_CU(EPI, NTV, 3);             \
    } while (0)
#define TG_CU_NT(E)                       \
    do {                                  \
        if (nt) TG_CU_PD(E, true);        \
        else TG_CU_PD(E, false);          \
    } while (0)
    TG_EPI_DISPATCH(epi, TG_CU_NT);
#undef TG_CU_NT
    return hipErrorInvalidValue;
#undef TG_CU_PD
#undef TG_CU
}

int igemm_cu_stats_grid(const ConvGeom& g) {
    const int nblocks = (g.M + 15) / 16;
    return nblocks < 256 ? nblocks : 256;
}

hipError_t launch_igemm_cu_stats(const ConvGeom& g, int nwaves, int pd, const void* x,
                                 const void* w, double* stats, hipStream_t s) {
    if (!igemm_cu_serves(g) || g.out8 || g.res || nwaves < 1 || nwaves > kCuStatsThreads / 64 ||
        nwaves % (g.C_out / kCuCW) != 0)
        return hipErrorInvalidValue;
    const int grid = igemm_cu_stats_grid(g);
    if (grid == 0) return hipSuccess;
    if (pd <= 1)
        return launch_cu_t<EPI_IDENTITY, false, 1, false, false, true>(g, grid, nwaves, x, w,
                                                                      nullptr, nullptr, nullptr, s,
                                                                      stats);
    if (pd == 2)
        return launch_cu_t<EPI_IDENTITY, false, 2, false, false, true>(g, grid, nwaves, x, w,
                                                                      nullptr, nullptr, nullptr, s,
                                                                      stats);
    return launch_cu_t<EPI_IDENTITY, false, 3, false, false, true>(g, grid, nwaves, x, w, nullptr,
                                                                  nullptr, nullptr, s, stats);
}

}  // namespace tg
