// igemm_band.hip -- conv2d_bn_silu_igemm for stride-1 convolutions with
// C_in % 64 == 0 and 64 or 128 output channels (the 3x3 and 7x7 body
// layers): one workgroup computes a band of consecutive output pixels of one
// image for every output channel. Opt-in (tuning key band=1): on those
// layers it runs level with the patch-staged kernel (3x3) or slower (7x7).
//
// The operation is that of igemm.hip ("Fusing an Epilogue", teenygrad docs,
// "The shape of it": the K loop on the matrix cores leaves the output tile in
// registers; BatchNorm scale/shift and the activation are applied there, then
// one store). The design keeps the K loop free of workgroup barriers:
//   * Four waves, one per SIMD, each with a 64-channel x 112-pixel register
//     tile (4 x 7 blocks of 16x16x32 MFMA). Two K groups split every
//     64-channel chunk into halves; their partial tiles are summed through
//     LDS once, at the end.
//   * A tile is all output channels of 112 (C_out = 128) or 224 (C_out = 64)
//     consecutive pixels; the input rows it touches (all C_in channels,
//     zero-padded at the image border) are loaded into LDS at kernel start
//     by all four waves, as 64-channel slices of 160 bytes per pixel; a tap
//     (r, s) moves a pixel fragment's address by a wave-uniform
//     (r*PW + s)*160. One loader wave streaming the rows stage by stage
//     instead kept too few loads in flight and ran 30% slower.
//   * Each wave streams its own filter rows and K half into a private LDS
//     ring (direct-to-LDS loads, three chunks deep). Four lanes fetch one
//     contiguous 64-byte row segment, and the rotated slot order makes every
//     fragment read touch each bank once per 16 lanes. Nothing else reads
//     the ring, so the wave's own load count orders it. (Filter fragments
//     loaded from the OHWI filter straight into registers touch 16 cache
//     lines per load and ran 15-25% slower.)
//   * Fragment reads for chunk k+1 are interleaved with chunk k's MFMAs; an
//     odd chunk count runs one step on zero-filled filter chunks, so every
//     step has the same shape.
//   * The epilogue: each K group hands the other the partial sums of the
//     pixel blocks it does not own; ownership is a compile-time fact per
//     group, so the partner reads of a block row go out together. BatchNorm
//     constants come from LDS; the fp16 tile is staged in LDS and written as
//     one contiguous range of y with non-temporal 16-byte stores.
#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {
namespace {

constexpr int kBdFM = 7;          // 16-pixel blocks per wave
constexpr int kBdFN = 4;          // 16-channel blocks per wave
constexpr int kBdPx = 160;        // LDS bytes per pixel of a 64-channel slice
constexpr int kBdPxPerDma = 6;    // slice pixels per direct-to-LDS instruction (60 lanes)
constexpr int kBdRing = 3;        // filter chunks in each compute wave's LDS ring
constexpr int kBdThreads = 256;
constexpr int kBdLds = 160 * 1024;

struct BandArgs {
    ConvGeom g;
    int tiles_per_img;
    int PW;        // patch columns, Q + kw - 1
    int PRmax;     // patch rows allocated per 64-channel slice
    int ipr;       // direct-to-LDS instructions per patch row slice
    int steps;     // K steps: kh * kw * C_in / 64
    int ring_off;  // LDS byte offsets: epilogue space (after the BatchNorm constants)
    int patch_off;
    int wring_off; // the compute waves' filter rings
};

template <int N>
__device__ __forceinline__ void bd_wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void bd_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ u32x4_t bd_rsrc(const void* base, unsigned bytes) {
    const unsigned long long a = (unsigned long long)base;
    u32x4_t r;
    r[0] = (unsigned)a;
    r[1] = (unsigned)(a >> 32) & 0xffffu;
    r[2] = bytes;  // reads at or past num_records return zeros
    r[3] = 0x00020000u;
    return r;
}

// Direct-to-LDS loads: lane l's 16 (4) bytes land at lds + 16*l (4*l).
// Inline assembly, so the compiler adds no wait of its own; completion is
// ordered by the explicit vmcnt waits and barriers of the caller.
__device__ __forceinline__ void bd_dma16(u32x4_t rsrc, unsigned voff, unsigned lds) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds)
                 : "memory");
}
__device__ __forceinline__ void bd_dma4(u32x4_t rsrc, unsigned voff, unsigned lds) {
    asm volatile("buffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds)
                 : "memory");
}

// 16-byte LDS read whose completion is the caller's explicit lgkmcnt wait.
__device__ __forceinline__ half8_t bd_lds16(unsigned addr) {
    half8_t r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr) : "memory");
    return r;
}

template <int V>
struct BdInt {
    static constexpr int value = V;
};

template <int WN, int EPI>
__global__ __launch_bounds__(kBdThreads, 1) void conv2d_bn_silu_igemm_band(
    const f16* __restrict__ x, const f16* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, f16* __restrict__ y, BandArgs a) {
    constexpr int WM = 2 / WN;
    constexpr int FM = kBdFM, FN = kBdFN;
    constexpr int TM = 16 * FM * WM;         // pixels per tile
    constexpr int CO = 64 * WN;              // output channels
    constexpr int OROW = CO + 8;             // output tile row (halves)
    extern __shared__ __attribute__((aligned(16))) unsigned char bd_smem[];
    const ConvGeom& g = a.g;

    const int tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    const int n = tile / a.tiles_per_img;
    const int PQ = g.P * g.Q;
    const int t0 = (tile - n * a.tiles_per_img) * TM;  // first output pixel in the image
    const int t1 = imin(t0 + TM, PQ);
    const int p_first = t0 / g.Q;
    const int orows = (t1 - 1) / g.Q - p_first + 1;
    const int PR = orows + g.kh - 1;                    // patch rows of this tile
    const int KK = g.kh * g.kw;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const unsigned lds0 = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)bd_smem));
    const unsigned patch = lds0 + (unsigned)a.patch_off;

    const int kg = wave & 1;                            // K half of every chunk
    const int wn = WN == 2 ? wave >> 1 : 0;
    const int wm = WN == 2 ? 0 : wave >> 1;
    const int lr = lane & 15, lg = lane >> 4;

    // Prologue: the whole patch, then the BatchNorm constants (wave 0).
    // Patch instruction t fills pixels 6j..6j+5 of row slice t / ipr
    // (slice = cc*PR + pr: patch row pr, channels 64cc..64cc+63); lane l
    // takes pixel 6j + l/10, piece l%10 (pieces 8 and 9 are the zero pad of
    // the 160-byte stride); wave w issues t = w, w+4, ... All four waves
    // issue them: one wave alone keeps too few loads in flight to stream the
    // rows at the rate the K loop would consume them.
    {
        const int T = (g.C_in / 64) * PR * a.ipr;
        const u32x4_t xrs =
            bd_rsrc(x, (unsigned)g.N * (unsigned)g.H * (unsigned)g.W * (unsigned)g.C_in * 2u);
        const int pl_px = lane / 10, pl_piece = lane - (lane / 10) * 10;
        for (int t = wave; t < T; t += 4) {
            const int slice = t / a.ipr, j = t - (t / a.ipr) * a.ipr;
            const int cc = slice / PR, pr = slice - (slice / PR) * PR;
            const int px = kBdPxPerDma * j + pl_px;
            const int ih = p_first - g.pad + pr, iw = px - g.pad;
            const bool data = pl_piece < 8 && (unsigned)ih < (unsigned)g.H &&
                              (unsigned)iw < (unsigned)g.W;
            const unsigned off =
                data ? (unsigned)(((((n * g.H + ih) * g.W + iw) * g.C_in) + cc * 64 + pl_piece * 8) * 2)
                     : 0x80000000u;
            const unsigned dst =
                patch + (unsigned)(((cc * a.PRmax + pr) * a.PW + kBdPxPerDma * j) * kBdPx);
            if (lane < 10 * kBdPxPerDma && px < a.PW) bd_dma16(xrs, off, dst);
        }
    }
    if (EPI != EPI_IDENTITY && wave == 0) {
#pragma unroll
        for (int c = 0; c < CO / 64; ++c) {
            bd_dma4(bd_rsrc(scale, (unsigned)g.C_out * 4u), (unsigned)((c * 64 + lane) * 4),
                    lds0 + (unsigned)(c * 256));
            bd_dma4(bd_rsrc(bias, (unsigned)g.C_out * 4u), (unsigned)((c * 64 + lane) * 4),
                    lds0 + (unsigned)(CO * 4 + c * 256));
        }
    }

    // A operand (filter): every compute wave streams its own rows and K half
    // of each chunk into a private ring of kBdRing slots in LDS (no other
    // wave reads them, so no barrier orders them; the wave's own
    // vector-memory count does). A slot holds FN fragments of 1 KB: 16 rows
    // (filter rows wn*64 + 16i ..) x 64 bytes (channels 32kg .. 32kg+31 of
    // the chunk's 64-channel slice). Row lr, piece p sits in 16-byte slot
    // 4*lr + ((p + lr/4) & 3): the four lanes of one row fetch one
    // contiguous 64-byte segment, and a fragment read (lane lr + 16*lg takes
    // row lr, piece lg) touches every bank once per 16 lanes. Chunk k = tap
    // k % KK of slice k / KK sits at byte (tap*C_in + 64*slice)*2 of every
    // OHWI row; chunks past the last read zeros.
    constexpr int R = kBdRing;
    const u32x4_t wrs = bd_rsrc(w, (unsigned)g.C_out * (unsigned)g.K * 2u);
    unsigned wsrc[FN];
    {
        const int row = lane >> 2;
        const int piece = ((lane & 3) - (row >> 2)) & 3;
#pragma unroll
        for (int i = 0; i < FN; ++i)
            wsrc[i] = (unsigned)(((wn * 64 + i * 16 + row) * g.K + kg * 32 + piece * 8) * 2);
    }
    const unsigned wring = lds0 + (unsigned)a.wring_off + (unsigned)(wave * R * FN * 1024);
    int wk = 0, wtap = 0, wslot = 0;
    unsigned wkoff = 0;  // (wtap*C_in + 64*slice)*2 of chunk wk
    auto issue_w = [&]() {  // chunk wk into slot wk % R, then advance wk
        const unsigned koff = wk < a.steps ? wkoff : 0x80000000u;
        const unsigned dst = wring + (unsigned)(wslot * FN * 1024);
#pragma unroll
        for (int i = 0; i < FN; ++i) bd_dma16(wrs, wsrc[i] + koff, dst + (unsigned)(i * 1024));
        ++wk;
        if (++wslot == R) wslot = 0;
        wkoff += (unsigned)(g.C_in * 2);
        if (++wtap == KK) {
            wtap = 0;
            wkoff -= (unsigned)(KK * g.C_in * 2) - 128u;
        }
    };
#pragma unroll
    for (int k = 0; k < R; ++k) issue_w();  // chunks 0 .. R-1

    // Fragment offsets. A: fragment i of a slot. B (pixels, from the
    // patch): pixel block j of this wave, channels 32kg + 8lg.. of the
    // slice, at tap (0, 0) of slice 0.
    const unsigned ab = (unsigned)((lr * 4 + ((lg + (lr >> 2)) & 3)) * 16);
    int bb[FM];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        int m = t0 + (wm * FM + j) * 16 + lr;
        if (m > t1 - 1) m = t1 - 1;  // past the image: any valid pixel, result unused
        const int p = m / g.Q, q = m - (m / g.Q) * g.Q;
        bb[j] = ((p - p_first) * a.PW + q) * kBdPx + kg * 64 + lg * 16;
    }
    // LDS bases of the chunk whose fragments are read next: its ring slot
    // and the patch at its tap and slice, advanced one chunk at a time (taps
    // s, then r, then the 64-channel slice). Past the last chunk the patch
    // base stays put (valid reads) while the slot moves on to zero-filled
    // filter chunks, so those MFMAs add nothing.
    struct Cursor {
        int k, r, s, slot;
        unsigned pd;
    };
    const unsigned slice_bytes = (unsigned)(a.PRmax * a.PW * kBdPx);
    auto advance = [&](Cursor& c) {
        if (++c.slot == R) c.slot = 0;
        if (c.k + 1 >= a.steps) return;
        ++c.k;
        c.pd += kBdPx;
        if (++c.s == g.kw) {
            c.s = 0;
            c.pd += (unsigned)((a.PW - g.kw) * kBdPx);
            if (++c.r == g.kh) {
                c.r = 0;
                c.pd += slice_bytes - (unsigned)(g.kh * a.PW * kBdPx);
            }
        }
    };
    struct Frags {
        half8_t a[FN], b[FM];
    };
    auto frag_addr_a = [&](const Cursor& c, int i) {
        return wring + (unsigned)(c.slot * FN * 1024 + i * 1024) + ab;
    };
    // Wait for every outstanding fragment read; the registers pass through
    // empty asm statements first so that the reads count as consumed here.
    auto frag_wait = [&](Frags& F) {
#pragma unroll
        for (int i = 0; i < FN; ++i) asm volatile("" : "+v"(F.a[i]));
#pragma unroll
        for (int j = 0; j < FM; ++j) asm volatile("" : "+v"(F.b[j]));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };

    float4_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};

    Frags F0, F1;
    Cursor cur = {0, 0, 0, 0, patch};
    // The patch, the constants and chunk 0 have landed once only chunks
    // 1 .. R-1 may still be in flight (the barrier covers the patch rows
    // other waves loaded).
    bd_wait_vm<(R - 1) * FN>();
    bd_barrier();
#pragma unroll
    for (int i = 0; i < FN; ++i) F0.a[i] = bd_lds16(frag_addr_a(cur, i));
#pragma unroll
    for (int j = 0; j < FM; ++j) F0.b[j] = bd_lds16(cur.pd + (unsigned)bb[j]);
    advance(cur);
    frag_wait(F0);

    // Step k: chunk k's fragments are in registers (C), so its slot takes
    // chunk k+R; chunk k+1 has landed once only chunks k+2 .. k+R are in
    // flight. Its fragments (N) are read during the first FN + FM MFMAs of
    // chunk k. No barrier: the patch is read-only and the ring is private.
    auto step = [&](Frags& C, Frags& N) {
        issue_w();
        bd_wait_vm<(R - 1) * FN>();
#pragma unroll
        for (int f = 0; f < FN * FM; ++f) {
            const int i = f / FM, j = f % FM;
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(C.a[i], C.b[j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (f < FN) N.a[f] = bd_lds16(frag_addr_a(cur, f));
            else if (f < FN + FM) N.b[f - FN] = bd_lds16(cur.pd + (unsigned)bb[f - FN]);
            __builtin_amdgcn_sched_barrier(0);
        }
        advance(cur);
        frag_wait(N);
    };
    // Pairs of steps; an odd count runs one step past the last chunk, whose
    // filter fragments are zeros.
    int k = 0;
    do {
        step(F0, F1);
        step(F1, F0);
        k += 2;
    } while (k < a.steps);

    // ---- epilogue: the ring's last (zero) chunks land before the patch and
    // ring space is reused.
    bd_wait_vm<0>();
    bd_barrier();

    // K-group reduction: group 0 owns pixel blocks j < JH, group 1 the rest;
    // each hands its partial sums of the other group's blocks over through
    // LDS (slot = wave*16 + index among the handed-over blocks), then adds
    // its partner's to its owned blocks, applies BatchNorm and the
    // activation and writes the fp16 result into the output tile. Ownership
    // is a compile-time fact inside `body`, so all partner reads of a block
    // row go out before one wait.
    constexpr int JH = (FM + 1) / 2;
    float4_t* red = (float4_t*)(bd_smem + a.ring_off);
    f16* out = (f16*)(bd_smem + a.ring_off + 4 * 16 * 1024);
    const float* bn = (const float*)bd_smem;
    const int part = wave ^ 1;  // the other K group of this tile slice
    auto body = [&](auto kgc) {
        constexpr int KG = decltype(kgc)::value;
        constexpr int J0 = KG == 0 ? 0 : JH, J1 = KG == 0 ? JH : FM;  // owned blocks
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            if (j >= J0 && j < J1) continue;
            const int jj = KG == 0 ? j - JH : j;
#pragma unroll
            for (int i = 0; i < FN; ++i) red[(wave * 16 + jj * FN + i) * 64 + lane] = acc[i][j];
        }
        bd_barrier();
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int o = wn * 64 + i * 16 + lg * 4;  // 4 channels of this lane
            float4_t pv[J1 - J0];
#pragma unroll
            for (int j = J0; j < J1; ++j) pv[j - J0] = red[(part * 16 + (j - J0) * FN + i) * 64 + lane];
            const float4_t sc4 = *(const float4_t*)(bn + o);
            const float4_t bi4 = *(const float4_t*)(bn + CO + o);
            float sc[4], bi[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sc[e] = EPI == EPI_IDENTITY ? 0.0f : epi_scale<EPI>(sc4[e]);
                bi[e] = EPI == EPI_IDENTITY ? 0.0f : epi_scale<EPI>(bi4[e]);
            }
#pragma unroll
            for (int j = J0; j < J1; ++j) {
                const float4_t v = acc[i][j] + pv[j - J0];
                const int px = (wm * FM + j) * 16 + lr;
                half4_t h;
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = (f16)epilogue<EPI>(v[e], sc[e], bi[e]);
                *(half4_t*)(out + px * OROW + o) = h;
            }
        }
    };
    if (kg == 0) body(BdInt<0>{});
    else body(BdInt<1>{});
    bd_barrier();

    // The tile is one contiguous range of y: TM pixels x CO channels.
    {
        constexpr int CV = CO / 8;
        const int rows = t1 - t0;
        const long long ybase = ((long long)n * PQ + t0) * CO;
        for (int v = threadIdx.x; v < rows * CV; v += kBdThreads) {
            const int px = v / CV, c8 = v - (v / CV) * CV;
            store_y8<true>(y, ybase + (long long)v * 8, *(const half8_t*)(out + px * OROW + c8 * 8),
                           g.out8, g.res);
        }
    }
}

struct BandPlan {
    int WN, tiles, lds;
    BandArgs a;
};

// Output rows a tile of TM pixels starting at a multiple of TM can span.
int band_orows_max(const ConvGeom& g, int TM) {
    const int PQ = g.P * g.Q;
    int worst = 0;
    for (int t0 = 0; t0 < PQ; t0 += TM) {
        const int t1 = t0 + TM < PQ ? t0 + TM : PQ;
        const int rows = (t1 - 1) / g.Q - t0 / g.Q + 1;
        if (rows > worst) worst = rows;
    }
    return worst;
}

// Plan the tile and the LDS layout for g; false when the kernel does not
// serve the shape.
bool band_plan(const ConvGeom& g, BandPlan* bp) {
    if (g.stride != 1 || g.C_in % 64 != 0 || (g.C_out != 64 && g.C_out != 128)) return false;
    const long long xbytes = 2LL * g.N * g.H * g.W * g.C_in, wbytes = 2LL * g.C_out * g.K;
    if (xbytes >= (1LL << 31) || wbytes >= (1LL << 31)) return false;
    BandPlan p;
    p.WN = g.C_out / 64;
    const int TM = 16 * kBdFM * (2 / p.WN);
    const int PQ = g.P * g.Q;
    const int tpi = (PQ + TM - 1) / TM;
    BandArgs& A = p.a;
    A.g = g;
    A.tiles_per_img = tpi;
    A.PW = g.Q + g.kw - 1;
    A.PRmax = band_orows_max(g, TM) + g.kh - 1;
    A.ipr = (A.PW + kBdPxPerDma - 1) / kBdPxPerDma;
    const int cch = g.C_in / 64;
    A.steps = g.kh * g.kw * cch;
    const int bn_bytes = 2 * g.C_out * 4;
    A.ring_off = (bn_bytes + 15) / 16 * 16;
    const long long patch_bytes = (long long)cch * A.PRmax * A.PW * kBdPx;
    A.patch_off = A.ring_off;
    A.wring_off = (int)(A.patch_off + patch_bytes);
    const long long main_bytes = A.wring_off + 4LL * kBdRing * kBdFN * 1024;
    // Epilogue: 4 waves x 16 handed-over blocks of 1 KB, then the fp16 tile.
    const long long epi_bytes = A.ring_off + 4 * 16 * 1024 + (long long)TM * (g.C_out + 8) * 2;
    const long long lds = main_bytes > epi_bytes ? main_bytes : epi_bytes;
    if (lds > kBdLds) return false;
    p.tiles = g.N * tpi;
    p.lds = (int)lds;
    *bp = p;
    return true;
}

template <int WN>
hipError_t band_launch_t(const BandPlan& p, int epi, const void* x, const void* w,
                         const float* scale, const float* bias, void* y, hipStream_t s) {
    auto k = conv2d_bn_silu_igemm_band<WN, EPI_FUSED>;
#define TG_K(E) k = conv2d_bn_silu_igemm_band<WN, E>
    TG_EPI_DISPATCH(epi, TG_K);
#undef TG_K
    hipError_t e = ensure_dynamic_lds((const void*)k, (size_t)p.lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(p.tiles), dim3(kBdThreads), p.lds, s, (const f16*)x, (const f16*)w, scale,
                       bias, (f16*)y, p.a);
    return hipGetLastError();
}

}  // namespace

bool igemm_band_serves(const ConvGeom& g) {
    BandPlan p;
    return band_plan(g, &p);
}

void igemm_band_describe(const ConvGeom& g, int* tile_px, int* tiles, int* lds) {
    BandPlan p;
    if (!band_plan(g, &p)) {
        *tile_px = *tiles = *lds = 0;
        return;
    }
    *tile_px = 16 * kBdFM * (2 / p.WN);
    *tiles = p.tiles;
    *lds = p.lds;
}

hipError_t launch_igemm_band(const ConvGeom& g, int epi, const void* x, const void* w,
                             const float* scale, const float* bias, void* y, hipStream_t s) {
    BandPlan p;
    if (!band_plan(g, &p) || epi < 0 || epi >= kNumEpilogues) return hipErrorInvalidValue;
    return p.WN == 2 ? band_launch_t<2>(p, epi, x, w, scale, bias, y, s)
                     : band_launch_t<1>(p, epi, x, w, scale, bias, y, s);
}

}  // namespace tg
