// stem.hip -- conv2d_bn_silu for the network stem: 3x3 filter, stride 2,
// padding 1, three input channels (RGB), up to 64 output channels, even
// image width. HBM-bound (x read once, y written once).
//
// Same operation as the other fused kernels ("Fusing an Epilogue", teenygrad
// docs, "The shape of it": reduction on the matrix cores, BatchNorm + SiLU on
// the accumulators, one store).
//
// K layout. With three channels the three input pixels of one filter row
// (2q-1, 2q, 2q+1) are nine contiguous halves of an NHWC row. A window that
// starts one pixel earlier (pixel 2q-2, 12(q-1) bytes into the row) is
// 4-byte aligned and holds those nine values at halves 3..11 of a 16-half
// K-slot; the slot's other halves meet zero filter weights. One filter row
// is one slot, the K of one 32x32x16 MFMA: three MFMAs per 32 pixels and 32
// output channels (MFMA rows = filter channels, columns = pixels; lane
// (lc, hl) supplies window half hl of pixel lc).
//
// Data flow. A workgroup is one loader wave plus four compute waves and
// walks bands of R output rows of one image. The loader copies the band's
// 2R+1 input rows (those inside the image: a contiguous byte range of x) into
// LDS with direct-to-LDS loads of whole aligned 16-byte pieces, starting at
// the range's first byte rounded down to 16 (an earlier design that loaded
// each window straight from memory stalled the texture-data path on the L1
// with its overlapping misaligned 16-byte accesses). Rows outside the image
// are the zero padding: the compute waves skip them. Three band buffers keep
// up to two bands in flight; one workgroup barrier per band hands a buffer
// over. The loader only loads, so its waits are exact and the compute waves'
// stores are never waited for. Compute waves take 32-pixel groups of the
// band, read each window half as dwords from LDS, run the MFMAs and the
// epilogue, and store the group's 32 x C_out halves (contiguous in y)
// through a small LDS tile as whole 16-byte pieces. A lane keeps its pixel's
// row and column from one group to the next by adding (no division in the
// loop): the loop is VALU-bound, and per-group index arithmetic was most of
// it. Every half of the window that meets a zero weight (pixel 2q-2, and
// halves 12-15) is masked to zero, as are the padding pixel -1 (q = 0) and
// padding rows: the result never depends on an input outside the receptive
// field, Inf and NaN included. The second window half never reads past its
// row's end: its last 8 bytes are masked, not read from the next row.
#include <stdlib.h>

#include <type_traits>

#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {
namespace {

constexpr int kStemBands = 3;  // band buffers in LDS

template <int N>
__device__ __forceinline__ void stem_wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void stem_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16-byte direct-to-LDS buffer load (lane l -> lds + 16*l; offsets at or past
// num_records read as zeros); ordered by explicit vmcnt waits.
__device__ __forceinline__ void stem_dma16(u32x4_t rsrc, unsigned voff, unsigned lds) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds)
                 : "memory");
}

// Band buffer bytes: 2R+1 input rows, the up to 12 bytes that the
// rounded-down start adds and 20 bytes that the last window may read past
// its row (masked), rounded up to whole 1 KB load instructions.
__host__ __device__ inline int stem_band_bytes(int W, int R) {
    const int b = (2 * R + 1) * W * 6 + 32;
    return (b + 1023) / 1024 * 1024;
}

// STATS > 0 (training mode, one 32-channel slice; the number of 8-channel
// blocks whose statistics a lane keeps, C_out / 8, so that no registers hold
// channels past C_out): instead of the epilogue and the stores, each lane
// sums d = acc - shift and d^2 over its pixels (one shift per channel: that
// channel's conv output at the middle pixel of image 0, so that the sum of
// squares does not cancel when the mean is far from 0), and the workgroup's
// (count, mean, squared deviations) triple per channel goes to
// stats[(blockIdx.x * C_out + c) * 3] after fixed-order merges (lanes, then
// waves), as in the 1x1 kernel.
template <int NB, int EPI, int LI, int STATS>
__global__ __launch_bounds__(320) void conv2d_bn_silu_stem(
    const f16* __restrict__ x, const f16* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, f16* __restrict__ y, ConvGeom g, int R, int nbands,
    double* __restrict__ stats) {
    static_assert(LI <= 31, "vmcnt range for two bands in flight");
    constexpr int kMaxC = 32 * NB;
    // Band buffers are LI KB each: every band load issues exactly LI 1 KB
    // instructions (the ones past the band's rows read zeros) so that the
    // loader's wait counts are exact, and they all land inside the buffer.
    constexpr int band_bytes = LI * 1024;
    extern __shared__ __attribute__((aligned(16))) unsigned char stem_smem[];
    // [16-byte margin][band buffers][4 x 32 x kMaxC output tiles]. The
    // margin keeps the first window of a row (12 bytes before the row)
    // inside the allocation; what it reads there is masked.
    f16* tiles = (f16*)(stem_smem + 16 + kStemBands * band_bytes);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bands_per_img = (g.P + R - 1) / R;
    const int rowb = g.W * 6;  // bytes per input row
    // Bands of this workgroup: blockIdx.x, + gridDim.x, ...
    const int nmine = (int)blockIdx.x < nbands ? (nbands - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;

    if (wave == 4) {
        // ---------------- loader wave ----------------
        const unsigned long long a = (unsigned long long)x;
        u32x4_t rs;
        rs[0] = (unsigned)a;
        rs[1] = (unsigned)(a >> 32) & 0xffffu;
        rs[2] = (unsigned)g.N * (unsigned)g.H * (unsigned)rowb;
        rs[3] = 0x00020000u;
        const unsigned base = __builtin_amdgcn_readfirstlane(
            (unsigned)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)stem_smem) + 16u);
        // Band k of this workgroup into buffer k % kStemBands: byte c of the
        // buffer is byte a0 + c of x, a0 the band's first in-image row start
        // rounded down to 16. Every call for one of the workgroup's bands
        // issues exactly LI loads (past the band's rows: zeros); past its
        // last band, none.
        auto issue = [&](int k) {
            if (k >= nmine) return;
            const int band = (int)blockIdx.x + k * (int)gridDim.x;
            const int n = band / bands_per_img, p0 = (band - n * bands_per_img) * R;
            const int ih0 = 2 * p0 - 1 < 0 ? 0 : 2 * p0 - 1;
            const int ih1 = 2 * p0 + 2 * R < g.H ? 2 * p0 + 2 * R : g.H;  // exclusive
            const unsigned a0 = (unsigned)((n * g.H + ih0) * rowb) & ~15u;
            const unsigned a1 = (unsigned)((n * g.H + ih1) * rowb);
            const unsigned dst = base + (unsigned)((k % kStemBands) * band_bytes);
#pragma unroll
            for (int i = 0; i < LI; ++i) {
                const unsigned c = (unsigned)((i * 64 + lane) * 16);
                const bool ok = a0 + c < a1;
                stem_dma16(rs, ok ? a0 + c : 0x80000000u, dst + (unsigned)(i * 1024));
            }
        };
        // Band 0 alone first: at launch every workgroup's first band would
        // otherwise share HBM with its second, and compute would start later
        // (requesting all three at once measured 6% slower on the 224x224
        // stem).
        issue(0);
        stem_wait_vmcnt<0>();
        stem_barrier();  // band 0 ready
        issue(1);
        issue(2);
        for (int k = 0; k < nmine; ++k) {
            if (k + 2 < nmine)
                stem_wait_vmcnt<LI>();  // band k+1 landed (band k+2 may be pending)
            else
                stem_wait_vmcnt<0>();
            stem_barrier();  // band k done by every compute wave
            issue(k + 3);  // into the buffer band k has just released
        }
        stem_wait_vmcnt<0>();
        return;
    }

    // ---------------- compute waves ----------------
    // 32x32x16 MFMA: lane (lc, hl) supplies K halves 8hl..8hl+7 of column lc
    // (pixel) and row lc (channel); accumulator i of a lane is channel
    // 8(i/4) + 4hl + i%4 of pixel lc.
    const int lc = lane & 31, hl = lane >> 5;
    // Filter slots: A[f][r] holds, for channel 32f + lc, K-slot halves
    // 8hl..8hl+7 of filter row r: slot half j carries w[o][r][s][c] at
    // j = 3 + 3s + c, else 0.
    half8_t A[NB][3];
#pragma unroll
    for (int f = 0; f < NB; ++f)
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int o = 32 * f + lc;
            const bool ook = o < g.C_out;
            const int wb = ((ook ? o : 0) * 3 + r) * 9;
            half8_t v;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = 8 * hl + e - 3;  // 0..8 inside the window: (s, c) = (j/3, j%3)
                const bool ok = ook && j >= 0 && j < 9;
                const f16 wv = w[wb + (j < 0 ? 0 : (j > 8 ? 8 : j))];
                v[e] = ok ? wv : (f16)0.0f;
            }
            A[f][r] = v;
        }
    float sc[NB][16], bi[NB][16];
#pragma unroll
    for (int f = 0; f < NB; ++f)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            epi_consts<EPI>(scale, bias, 32 * f + 8 * (i / 4) + 4 * hl + (i % 4), g.C_out, sc[f][i],
                            bi[f][i]);

    f16* tl = tiles + wave * 32 * kMaxC;
    // Statistics (STATS): lane (lc, hl) sees pixel lc of each of its groups
    // and channels 32f + 8(i/4) + 4hl + i%4 of accumulator f, element i.
    constexpr int SI = STATS > 0 ? 4 * STATS : 1;  // accumulator elements with statistics
    float st_shift[NB][SI], st_s1[NB][SI], st_s2[NB][SI];
    int st_n = 0;
    if constexpr (STATS) {
        // Channel 32f + lc's shift is its conv output at the middle pixel
        // of image 0: lane (lc, hl) multiplies its filter fragments A[f][r]
        // with the same window halves the main loop would read for that
        // pixel (three 16-byte windows from x, masked as there; four dword
        // loads each, all in flight together), and the two halves add up.
        // Images under 2 x 2 outputs take 0 (their values are few and the
        // padding keeps them spread). Then every lane takes the shifts of its
        // accumulators' channels.
        float own[NB];
#pragma unroll
        for (int f = 0; f < NB; ++f) own[f] = 0.0f;
        if (g.P >= 2 && g.Q >= 2) {
            const int pm = g.P / 2, qm = g.Q / 2;  // input rows 2pm-1.. and columns 2qm-1.. lie inside
            const long long xbytes = 6LL * g.N * g.H * g.W;
            const unsigned hmk = hl ? ~0u : 0u;
            const u32x4_t m = {hmk, hmk | 0xffff0000u, ~hmk, ~hmk};
            half8_t win[3];
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const int ih = 2 * pm - 1 + r;
                const long long a = (long long)ih * rowb + 12 * qm - 12 + 16 * hl;  // image 0
                u32x4_t u;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const long long ad = a + 4 * d;
                    const bool ok = ih < g.H && ad + 4 <= xbytes;
                    u[d] = ((const unsigned*)x)[ok ? ad / 4 : 0];
                    u[d] = ok ? u[d] : 0u;
                }
                win[r] = __builtin_bit_cast(half8_t, u & m);
            }
#pragma unroll
            for (int f = 0; f < NB; ++f) {
                float sum = 0.0f;
#pragma unroll
                for (int r = 0; r < 3; ++r)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        sum = __builtin_fmaf((float)win[r][e], (float)A[f][r][e], sum);
                own[f] = sum + __shfl_xor(sum, 32);
            }
        }
#pragma unroll
        for (int f = 0; f < NB; ++f)
#pragma unroll
            for (int i = 0; i < SI; ++i) {
                st_shift[f][i] = __shfl(own[f], 8 * (i / 4) + 4 * hl + (i % 4));
                st_s1[f][i] = st_s2[f][i] = 0.0f;
            }
    }
    // Window dwords that always meet zero weights: half 0 holds pixel 2q-2
    // (halves 0-2) before 2q-1 and 2q; half 1 holds 2q, 2q+1 (halves 8-11)
    // and nothing of use in halves 12-15.
    const unsigned hm = hl ? ~0u : 0u;
    const int hoff = 16 * hl - 12;  // window bytes from 12q in its row
    stem_barrier();  // band 0 ready
    for (int k = 0; k < nmine; ++k) {
        const int band = (int)blockIdx.x + k * (int)gridDim.x;
        const int n = band / bands_per_img, p0 = (band - n * bands_per_img) * R;
        const int rows = g.P - p0 < R ? g.P - p0 : R;
        // Input row ih sits at byte (ih - ih0) * rowb + shift of the buffer.
        const int ih0 = 2 * p0 - 1 < 0 ? 0 : 2 * p0 - 1;
        const int shift = ((n * g.H + ih0) * rowb) & 15;
        const unsigned char* bb = stem_smem + 16 + (k % kStemBands) * band_bytes + shift;
        const int npx = rows * g.Q;
        const int ngroups = (npx + 31) / 32;
        const long long m_base = ((long long)n * g.P + p0) * g.Q;  // first pixel of the band
        int pix = wave * 32 + lc;
        int pl = pix / g.Q;
        int q = pix - pl * g.Q;
        int ihr = 2 * (p0 + pl) - 1;    // input row of filter row 0
        int roff = (ihr - ih0) * rowb;  // its byte offset in the buffer (-rowb: row -1)
        int colb = 12 * q;
        // Bands touching a padding row (top of the image, or the bottom when
        // H is odd) check rows per lane; the others skip that code.
        auto walk = [&](auto edge_tag) {
            constexpr bool EDGE = decltype(edge_tag)::value;
            for (int grp = wave; grp < ngroups; grp += 4) {
                const bool pok = pix < npx;
                // Lanes past the band read a harmless in-buffer address.
                const int a = pok ? roff + colb + hoff : 16;
                const unsigned lm = q == 0 ? 0u : ~0u;  // q = 0: pixel -1 is padding
                const u32x4_t m = {hm, hm | (lm & 0xffff0000u), ~hm & lm, ~hm};
                half8_t b[3];
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    int at = a + r * rowb;
                    bool rok = true;
                    if (EDGE) {  // padding rows are not in the buffer (row -1 lies before it)
                        rok = (unsigned)(ihr + r) < (unsigned)g.H;
                        if (!rok) at = 16;
                    }
                    const unsigned* p32 = (const unsigned*)(bb + at);
                    u32x4_t u = {p32[0], p32[1], p32[2], p32[3]};
                    u &= m;
                    if (EDGE && !rok) u = (u32x4_t){0u, 0u, 0u, 0u};
                    b[r] = __builtin_bit_cast(half8_t, u);
                }
                float16_t acc[NB];
#pragma unroll
                for (int f = 0; f < NB; ++f) {
                    acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[f][0], b[0], (float16_t){}, 0, 0, 0);
                    acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[f][1], b[1], acc[f], 0, 0, 0);
                    acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[f][2], b[2], acc[f], 0, 0, 0);
                }
                if constexpr (STATS) {
                    st_n += pok ? 1 : 0;
                    // Lanes past the band (their window is any in-buffer
                    // data, their sums may not be finite) add +0: a bit mask
                    // rather than a select, which the compiler turned into a
                    // branch per element.
                    const unsigned pmask = pok ? ~0u : 0u;
#pragma unroll
                    for (int f = 0; f < NB; ++f)
#pragma unroll
                        for (int i = 0; i < SI; ++i) {
                            const float d = __builtin_bit_cast(
                                float, pmask & __builtin_bit_cast(unsigned, acc[f][i] - st_shift[f][i]));
                            st_s1[f][i] += d;
                            st_s2[f][i] = __builtin_fmaf(d, d, st_s2[f][i]);
                        }
                } else {
#pragma unroll
                for (int f = 0; f < NB; ++f)
#pragma unroll
                    for (int blk = 0; blk < 4; ++blk) {
                        const int c0 = 32 * f + 8 * blk;  // C_out % 8 == 0: whole blocks
                        if (c0 < g.C_out) {
                            half4_t h;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                h[e] = (f16)epilogue<EPI>(acc[f][4 * blk + e], sc[f][4 * blk + e],
                                                          bi[f][4 * blk + e]);
                            *(half4_t*)(tl + lc * g.C_out + c0 + 4 * hl) = h;
                        }
                    }
                asm volatile("" ::: "memory");
                __builtin_amdgcn_wave_barrier();
                asm volatile("" ::: "memory");
                // The group's 32 x C_out halves are contiguous in y.
                const int valid = npx - grp * 32 < 32 ? npx - grp * 32 : 32;
                const int pieces = valid * g.C_out / 8;
                const long long yg = (m_base + grp * 32) * g.C_out;  // first element of y
#pragma unroll
                for (int i = 0; i < (4 * kMaxC + 63) / 64; ++i) {
                    const int v = lane + 64 * i;
                    if (v < pieces) store_y8<true>(y, yg + v * 8, *(const half8_t*)(tl + v * 8), g.out8, g.res);
                }
                asm volatile("" ::: "memory");
                __builtin_amdgcn_wave_barrier();
                asm volatile("" ::: "memory");
                }  // !STATS
                // Next group of this wave: 128 pixels on.
                pix += 128;
                q += 128;
                colb += 12 * 128;
                while (q >= g.Q) {
                    q -= g.Q;
                    colb -= 12 * g.Q;
                    ihr += 2;
                    roff += 2 * rowb;
                }
            }
        };
        if (p0 == 0 || 2 * (p0 + rows) > g.H)
            walk(std::true_type{});
        else
            walk(std::false_type{});
        stem_barrier();  // band k consumed; band k+1 ready
    }
    if constexpr (STATS) {
        // Sums over the 32 lanes of each half (the 16 lanes of a DPP row,
        // then the other row of the half), every lane ending with its
        // half's totals; then the (count, mean, squared deviations) triple
        // in fp64.
        auto sum32 = [](float v) {
            v = row_sum16(v);
            return v + __shfl_xor(v, 16);
        };
        const float nh = sum32((float)st_n);  // pixels of the half: exact in fp32
        const double n0 = (double)nh;
        const double inv_n = nh > 0.0f ? 1.0 / n0 : 0.0;
        // Wave-local triples in the (now unused) output tiles: channel c of
        // wave v at ((v * kMaxC + c) * 3).
        double* wt = (double*)tiles;
#pragma unroll
        for (int f = 0; f < NB; ++f)
#pragma unroll
            for (int i = 0; i < SI; ++i) {
                // One channel at a time (the empty asm statements keep their
                // order): the sums and fp64 values of all of them would
                // otherwise be live at once and cost the kernel occupancy.
                asm volatile("" : "+v"(st_s1[f][i]), "+v"(st_s2[f][i]));
                const double s1 = sum32(st_s1[f][i]), s2 = sum32(st_s2[f][i]);
                const double mean = nh > 0.0f ? (double)st_shift[f][i] + s1 * inv_n : 0.0;
                double m2 = s2 - s1 * s1 * inv_n;
                m2 = m2 > 0.0 ? m2 : 0.0;
                const int c = 32 * f + 8 * (i / 4) + 4 * hl + (i % 4);
                if (lc == 0) {
                    double* dst = wt + (wave * kMaxC + c) * 3;
                    dst[0] = n0;
                    dst[1] = mean;
                    dst[2] = m2;
                }
                asm volatile("" ::"v"(mean), "v"(m2) : "memory");
            }
        stem_barrier();  // the loader wave has finished: the compute waves alone
        if (wave == 0 && lane < g.C_out) {
            double n = 0.0, mean = 0.0, m2 = 0.0;
            for (int v = 0; v < 4; ++v) {
                const double* src = wt + (v * kMaxC + lane) * 3;
                chan_merge(n, mean, m2, src[0], src[1], src[2]);
            }
            double* dst = stats + ((size_t)blockIdx.x * g.C_out + lane) * 3;
            dst[0] = n;
            dst[1] = mean;
            dst[2] = m2;
        }
    }
}

}  // namespace

int stem_rows(const ConvGeom& g) {
    // Enough rows that a band holds a few 32-pixel groups per compute wave.
    int R = (384 + g.Q - 1) / g.Q;
    if (R < 2) R = 2;
    if (R > 8) R = 8;
    if (R > g.P) R = g.P;
    while (R > 1 && stem_band_bytes(g.W, R) > 31 * 1024) --R;
    return R;
}

bool stem_rows_ok(const ConvGeom& g, int R) {
    return R >= 1 && R <= g.P && stem_band_bytes(g.W, R) <= 31 * 1024;
}

bool stem_serves(const ConvGeom& g) {
    return g.C_in == 3 && g.kh == 3 && g.kw == 3 && g.stride == 2 && g.pad == 1 &&
           g.W % 2 == 0 && g.C_out % 8 == 0 && g.C_out <= 64 && stem_rows_ok(g, 1) &&
           6LL * g.N * g.H * g.W < (1LL << 31);
}

int stem_grid(const ConvGeom& g, int wg_per_cu, int R) {
    const int bands = g.N * ((g.P + R - 1) / R);
    long long grid = 256LL * (wg_per_cu < 1 ? 1 : wg_per_cu);
    return grid > bands ? bands : (int)grid;
}

namespace {

// The stem kernel for (NB, EPI, STATS) with the band buffer size chosen
// from the image width and band rows.
template <int NB, int EPI, int STATS>
hipError_t stem_launch_li(const ConvGeom& g, int grid, int R, const void* x, const void* w,
                          const float* scale, const float* bias, void* y, double* stats,
                          hipStream_t s) {
    const int bands = g.N * ((g.P + R - 1) / R);
    const int li = stem_band_bytes(g.W, R) / 1024;
#define TG_STEM_K(LIV)                                                                        \
    do {                                                                                      \
        auto k = conv2d_bn_silu_stem<NB, EPI, LIV, STATS>;                                    \
        const size_t lds = 16 + (size_t)kStemBands * (LIV)*1024 + 4 * 32 * 32 * NB * 2;        \
        hipError_t e = ensure_dynamic_lds((const void*)k, lds);                               \
        if (e != hipSuccess) return e;                                                        \
        hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(320), lds, s, (const f16*)x,         \
                           (const f16*)w, scale, bias, (f16*)y, g, R, bands, stats);           \
        return hipGetLastError();                                                             \
    } while (0)
    if (li <= 4) TG_STEM_K(4);
    if (li <= 6) TG_STEM_K(6);
    if (li <= 8) TG_STEM_K(8);
    if (li <= 10) TG_STEM_K(10);
    if (li <= 12) TG_STEM_K(12);
    if (li <= 14) TG_STEM_K(14);
    if (li <= 16) TG_STEM_K(16);
    if (li <= 20) TG_STEM_K(20);
    if (li <= 24) TG_STEM_K(24);
    TG_STEM_K(31);
#undef TG_STEM_K
}

}  // namespace

hipError_t launch_stem(const ConvGeom& g, int wg_per_cu, int R, int epi, const void* x,
                       const void* w, const float* scale, const float* bias, void* y,
                       hipStream_t s) {
    if (!stem_serves(g) || !stem_rows_ok(g, R)) return hipErrorInvalidValue;
    const int grid = stem_grid(g, wg_per_cu, R);
    const int nb = (g.C_out + 31) / 32;
#define TG_STEM_1(E) return stem_launch_li<1, E, 0>(g, grid, R, x, w, scale, bias, y, nullptr, s)
#define TG_STEM_2(E) return stem_launch_li<2, E, 0>(g, grid, R, x, w, scale, bias, y, nullptr, s)
    if (nb == 1) TG_EPI_DISPATCH(epi, TG_STEM_1);
    TG_EPI_DISPATCH(epi, TG_STEM_2);
    return hipErrorInvalidValue;
#undef TG_STEM_2
#undef TG_STEM_1
}

bool stem_stats_serves(const ConvGeom& g) { return stem_serves(g) && g.C_out <= 32; }

// The statistics instance holds up to 127 registers for C_out <= 24 (four
// waves per SIMD: three workgroups per CU, as the inference kernel) and 151
// for C_out = 32 (three: two workgroups).
int stem_stats_wpc(const ConvGeom& g) { return g.C_out <= 24 ? 3 : 2; }

hipError_t launch_stem_stats(const ConvGeom& g, int R, const void* x, const void* w,
                             double* stats, hipStream_t s) {
    if (!stem_stats_serves(g) || !stem_rows_ok(g, R) || g.out8 || g.res)
        return hipErrorInvalidValue;
    const int grid = stem_grid(g, stem_stats_wpc(g), R);
#define TG_STEM_ST(CB)                                                                        \
    return stem_launch_li<1, EPI_IDENTITY, CB>(g, grid, R, x, w, nullptr, nullptr, nullptr, \
                                               stats, s)
    switch (g.C_out / 8) {  // C_out % 8 == 0, at most 32
        case 1: TG_STEM_ST(1);
        case 2: TG_STEM_ST(2);
        case 3: TG_STEM_ST(3);
        default: TG_STEM_ST(4);
    }
#undef TG_STEM_ST
}

}  // namespace tg
