// igemm_rw.hip -- conv2d_bn_silu_igemm, register-resident-weights variant for
// short reductions (K = kh*kw*C_in <= 64) and up to 256 output channels:
// the shape of a 1x1 channel-mixing convolution, which is HBM-bound (about
// 51 FLOP per byte, far below the MFMA ridge) and dominated by the y stores.
//
// Same operation as igemm.hip ("Fusing an Epilogue", teenygrad docs, "The
// shape of it": K-loop, then BatchNorm scale/shift and SiLU on the register
// tile, then one store), organised for a store-bound stream on gfx950:
//   * Workgroups are persistent and own one contiguous range of 16-pixel
//     blocks, so each writes y as one sequential stream.
//   * Wave specialisation. Vector loads and stores share one completion
//     counter on this architecture, so a wave that waits for a prefetched
//     load also waits for every store it issued before. The compute waves
//     therefore never load after their prologue; one extra wave per workgroup
//     only loads: it streams the im2col fragments of the coming rounds
//     straight into an LDS ring with direct-to-LDS buffer loads (no VGPRs;
//     lane l's 16 bytes land at offset 16*l, which is exactly the MFMA
//     operand layout; taps outside the image get an out-of-range offset,
//     which the buffer unit turns into zeros). RING rounds are in flight and
//     one workgroup barrier per round hands a stage over.
//   * Each compute wave holds its slice of the filter bank in VGPRs, already
//     in the MFMA row-operand layout, with the rows permuted so that the
//     accumulator of lane (r, g) holds 8 consecutive output channels of one
//     pixel: row i of fragment f computes channel
//         sigma(f, i) = 32*(f/2) + 8*(i/4) + 4*(f%2) + i%4.
//     BatchNorm + SiLU then run directly on the accumulators (the lane's
//     per-channel scale and bias live in registers for the whole kernel).
//   * The fp16 results of a 16-pixel block go through a small padded LDS
//     tile shared by the waves that computed its channel slices; after the
//     round barrier each of them stores its share of the tile as whole pixel
//     rows. A store instruction must cover full 128-byte lines of y: 64-byte
//     pieces cost about 40% of the write bandwidth on this part.
#include <stdlib.h>

#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {

// LDS write visibility for the other waves, then the workgroup barrier. No
// vector-memory wait: compute waves must not wait for their stores here.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most k*PER vector-memory operations of this wave are pending.
template <int PER, int MAXK>
__device__ __forceinline__ void wait_rounds_pending(int k) {
    static_assert(PER * (MAXK - 1) <= 63, "vmcnt range");
    switch (k) {
#define TG_CASE(i) \
    case i: if (i < MAXK) wait_vmcnt<(i < MAXK ? i * PER : 0)>(); break;
        TG_CASE(0) TG_CASE(1) TG_CASE(2) TG_CASE(3) TG_CASE(4) TG_CASE(5) TG_CASE(6)
        TG_CASE(7) TG_CASE(8) TG_CASE(9) TG_CASE(10) TG_CASE(11) TG_CASE(12) TG_CASE(13)
        TG_CASE(14) TG_CASE(15)
#undef TG_CASE
        default: wait_vmcnt<0>(); break;
    }
}

// Direct-to-LDS 16-byte buffer load (lane l's bytes land at lds + 16*l;
// offsets past num_records read as zeros), written as inline assembly so the
// compiler does not see an LDS write it must wait for: the caller orders it
// with explicit vmcnt waits. rsrc = {base_lo, base_hi, num_records, flags};
// lds must be wave-uniform.
__device__ __forceinline__ void lds_dma16(u32x4_t rsrc, unsigned voff, unsigned lds) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds)
                 : "memory");
}

__device__ __forceinline__ u32x4_t raw_buffer_rsrc(const void* base, unsigned bytes) {
    const unsigned long long a = (unsigned long long)base;
    u32x4_t r;
    r[0] = (unsigned)a;
    r[1] = (unsigned)(a >> 32) & 0xffffu;  // stride 0, no swizzle
    r[2] = bytes;
    r[3] = 0x00020000u;                    // same descriptor flags as the loader wave
    return r;
}

// Orders one wave's LDS writes before its following LDS reads of other lanes'
// data. The LDS executes a wave's operations in issue order, so only the
// compiler must be kept from moving accesses across this point. (A wavefront-
// scope fence would do the same but also waits for outstanding nontemporal
// stores.)
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// Output channel computed by row i of weight fragment f (see header).
__device__ __forceinline__ int rw_sigma(int f, int i) {
    return 32 * (f >> 1) + 8 * (i >> 2) + 4 * (f & 1) + (i & 3);
}

// NF: 16-row weight fragments per compute wave (even); KS: 32-deep k-steps;
// CSPLIT: compute waves sharing one 16-pixel block (each takes NF*16
// channels); NCW: compute waves per workgroup (plus one loader wave).
template <int NF, int KS, int CSPLIT, int NCW, int EPI, bool NT>
__global__ __launch_bounds__((NCW + 1) * 64) void conv2d_bn_silu_igemm_rw(
    const f16* __restrict__ x, const f16* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, f16* __restrict__ y, ConvGeom g, int nblocks) {
    static_assert(NF % 2 == 0 && NCW % CSPLIT == 0, "shape");
    constexpr int CW = NF * 16;          // channels per compute wave
    constexpr int BPR = NCW / CSPLIT;    // 16-pixel blocks per round
    constexpr int LPRND = BPR * KS;      // direct-to-LDS loads per round (per lane)
    constexpr int RING = 8;              // ring stages = rounds in flight
    constexpr int CT = CW * CSPLIT;      // channels per block tile
    constexpr int TROW = CT + 8;         // padded tile row (halves): rows start 4 banks apart
    constexpr int LPRW = CT / 8;         // lanes per tile row in the store phase
    constexpr int RPS = 64 / LPRW;       // tile rows per store instruction
    constexpr int SPW = 16 / RPS / CSPLIT;  // store instructions per wave per block
    static_assert(64 % LPRW == 0 && (16 / RPS) % CSPLIT == 0 && SPW >= 1, "store split");
    __shared__ __attribute__((aligned(16))) f16 ring[RING][BPR][KS][64 * 8];
    __shared__ __attribute__((aligned(16))) f16 tile[2][BPR][16 * TROW];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const half8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

    // Balanced contiguous split of the 16-pixel blocks over the workgroups;
    // round r gives block b_begin + BPR*r + w/CSPLIT to compute wave w.
    const int b_begin = (int)((long long)blockIdx.x * nblocks / gridDim.x);
    const int b_end = (int)((long long)(blockIdx.x + 1) * nblocks / gridDim.x);
    const int rounds = (b_end - b_begin + BPR - 1) / BPR;

    if (wave == NCW) {
        // ---------------- loader wave ----------------
        int tr[KS], ts[KS], tc[KS];
        bool tok[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            int k = 32 * s + 8 * lg;  // one filter tap: C_in % 8 == 0
            tok[s] = k < g.K;
            int tap = tok[s] ? k / g.C_in : 0;
            tc[s] = tok[s] ? k - tap * g.C_in : 0;
            tr[s] = tap / g.kw;
            ts[s] = tap - tr[s] * g.kw;
        }
        const int PQ = g.P * g.Q;
        // Whole x as one buffer; offsets past its end read as zeros.
        const unsigned xbytes = (unsigned)g.N * g.H * g.W * g.C_in * 2u;
        const __amdgpu_buffer_rsrc_t xr =
            __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)xbytes, 0x00020000);
        const unsigned kOut = 0x80000000u;  // > xbytes (x is below 2^31 bytes here)
        auto issue = [&](int r) {
            const int stage = r % RING;
#pragma unroll
            for (int wv = 0; wv < BPR; ++wv) {
                int blk = b_begin + BPR * r + wv;
                int m = blk * 16 + lr;
                bool mok = blk < b_end && m < g.M;
                int n = 0, p = 0, q = 0;
                if (mok) {
                    n = m / PQ;
                    int rem = m - n * PQ;
                    p = rem / g.Q;
                    q = rem - p * g.Q;
                }
                const int h0 = p * g.stride - g.pad, w0 = q * g.stride - g.pad;
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    int ih = h0 + tr[s], iw = w0 + ts[s];
                    bool ok = mok && tok[s] && (unsigned)ih < (unsigned)g.H &&
                              (unsigned)iw < (unsigned)g.W;
                    unsigned off =
                        ok ? (unsigned)((((n * g.H + ih) * g.W + iw) * g.C_in + tc[s]) * 2) : kOut;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        xr, (__attribute__((address_space(3))) void*)&ring[stage][wv][s][0], 16,
                        off, 0, 0, 0);
                }
            }
        };
        // Ramp the ring up: round 0 goes out alone (at kernel start every
        // workgroup fetches at once, and a deep first burst would queue each
        // workgroup's first round behind the others' later rounds), then at
        // most two more rounds per step until RING rounds are in flight.
        int issued = 0;
        if (rounds > 0) issue(issued++);
        if (issued < rounds) issue(issued++);
        if (rounds > 0) wait_rounds_pending<LPRND, RING>(issued - 1);
        lds_barrier();  // round 0 ready
        for (int r = 0; r < rounds; ++r) {
            // Stages r+1 .. issued-1 are loading; stage r is being consumed.
            for (int t = 0; t < 2 && issued < rounds && issued < r + RING; ++t) issue(issued++);
            // Round r+1's data must be in LDS before the barrier that ends round r.
            if (r + 1 < rounds) wait_rounds_pending<LPRND, RING>(issued - (r + 2));
            lds_barrier();
        }
        return;
    }

    // ---------------- compute waves ----------------
    const int slot = wave / CSPLIT;        // which block of the round
    const int c0 = (wave % CSPLIT) * CW;   // first output channel of this wave
    half8_t wf[NF][KS];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            int o = c0 + rw_sigma(f, lr), k = 32 * s + 8 * lg;
            wf[f][s] = (o < g.C_out && k < g.K) ? *(const half8_t*)(w + o * g.K + k) : zero8;
        }
    // Lane (lr, lg) owns channels c0 + 32*j + 8*lg + [0, 8) for j < NF/2.
    float sc[NF / 2][8], bi[NF / 2][8];
#pragma unroll
    for (int j = 0; j < NF / 2; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            epi_consts<EPI>(scale, bias, c0 + 32 * j + 8 * lg + e, g.C_out, sc[j][e], bi[j][e]);
        }
    const bool vec_store = (g.C_out & 7) == 0;
    const int cg = wave % CSPLIT;
    // Store phase: this lane copies 16 bytes of tile row (orow0 + RPS*i), at
    // channel ocs; rows [cg*RPS*SPW, (cg+1)*RPS*SPW) of each block are ours.
    const int ocs = (lane % LPRW) * 8;
    const int orow0 = cg * RPS * SPW + lane / LPRW;
    lds_barrier();  // ring stage 0 published

    for (int r = 0; r < rounds; ++r) {
        const int blk = b_begin + BPR * r + slot;
        f16* tl = &tile[r & 1][slot][0];
        if (blk < b_end) {
            half8_t xf[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s)
                xf[s] = *(const half8_t*)&ring[r % RING][slot][s][lane * 8];
            float4_t acc[NF];
#pragma unroll
            for (int f = 0; f < NF; ++f) acc[f] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int f = 0; f < NF; ++f)
                    acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[f][s], xf[s], acc[f], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < NF / 2; ++j) {
                half8_t h;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = (f16)epilogue<EPI>(acc[2 * j][e], sc[j][e], bi[j][e]);
                    h[4 + e] = (f16)epilogue<EPI>(acc[2 * j + 1][e], sc[j][4 + e], bi[j][4 + e]);
                }
                *(half8_t*)(tl + lr * TROW + c0 + 32 * j + 8 * lg) = h;
            }
        }
        lds_barrier();  // tiles of round r complete; ring stage r+1 ready
        if (blk < b_end) {
#pragma unroll
            for (int i = 0; i < SPW; ++i) {
                const int row = orow0 + RPS * i;
                const int m = blk * 16 + row;
                const half8_t v = *(const half8_t*)(tl + row * TROW + ocs);
                if (m < g.M && ocs < g.C_out) {
                    if (vec_store) {
                        store_y8<NT>(y, m * g.C_out + ocs, v, g.out8, g.res);
                    } else {
                        for (int e = 0; e < 8; ++e)
                            if (ocs + e < g.C_out) store_y1(y, m * g.C_out + ocs + e, v[e], g.out8, g.res);
                    }
                }
            }
        }
    }
}

// Streaming variant of the same computation: independent wavefronts, no
// loader wave, no workgroup barrier. Each wavefront owns one 16*NF-channel
// slice of the filter bank (in VGPRs, rows permuted by rw_sigma) and walks
// its own sequence of 16-pixel blocks: it fetches the block's im2col
// fragment straight into the MFMA column-operand registers one block ahead,
// runs NF*KS MFMAs, applies BatchNorm + SiLU on the accumulators, transposes
// the fp16 result through a wave-private LDS tile and stores whole 128-byte
// pieces of each pixel row. With four or more such wavefronts per SIMD, the
// waits on the shared load/store counter of one wavefront are covered by the
// others.
template <int NF, int KS, int EPI, bool NT, bool XDMA, int PD>
__global__ __launch_bounds__(256) void conv2d_bn_silu_igemm_stream(
    const f16* __restrict__ x, const f16* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, f16* __restrict__ y, ConvGeom g, int nblocks, int ngroups) {
    static_assert(NF % 2 == 0, "fragment pairs");
    constexpr int CW = NF * 16;       // channels per wavefront slice
    constexpr int TROW = CW + 8;      // padded tile row (halves)
    constexpr int LPRW = CW / 8;      // lanes per tile row when storing
    constexpr int RPS = 64 / LPRW;    // tile rows per store instruction
    static_assert(64 % LPRW == 0 && 16 % RPS == 0, "store split");
    __shared__ __attribute__((aligned(16))) f16 tile[4][16 * TROW];
    // Full-line x staging (XDMA): per wave PD buffers of 16 pixels x 64 k,
    // block it + PD fetched into the buffer block it was read from.
    static_assert(!XDMA || (PD >= 1 && 4 * PD - 2 <= 63), "prefetch depth");
    __shared__ __attribute__((aligned(16))) f16 xst[XDMA ? 4 : 1][XDMA ? PD : 1][16 * 64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const half8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const int gw = blockIdx.x * 4 + wave;
    const int cg = gw % ngroups;
    const int stream = gw / ngroups, nstreams = (gridDim.x * 4) / ngroups;
    const int c0 = cg * CW;
    if (stream >= nstreams) return;  // grid*4 is a multiple of ngroups; never taken

    half8_t wf[NF][KS];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            int o = c0 + rw_sigma(f, lr), k = 32 * s + 8 * lg;
            wf[f][s] = (o < g.C_out && k < g.K) ? *(const half8_t*)(w + o * g.K + k) : zero8;
        }
    float sc[NF / 2][8], bi[NF / 2][8];
#pragma unroll
    for (int j = 0; j < NF / 2; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            epi_consts<EPI>(scale, bias, c0 + 32 * j + 8 * lg + e, g.C_out, sc[j][e], bi[j][e]);
        }
    int tr[KS], ts[KS], tc[KS];
    bool tok[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        int k = 32 * s + 8 * lg;  // one filter tap: C_in % 8 == 0
        tok[s] = k < g.K;
        int tap = tok[s] ? k / g.C_in : 0;
        tc[s] = tok[s] ? k - tap * g.C_in : 0;
        tr[s] = tap / g.kw;
        ts[s] = tap - tr[s] * g.kw;
    }
    const int PQ = g.P * g.Q;
    auto fetch = [&](int blk, half8_t* xf) {
        int m = blk * 16 + lr;
        bool mok = blk < nblocks && m < g.M;
        int n = 0, p = 0, q = 0;
        if (mok) {
            n = m / PQ;
            int rem = m - n * PQ;
            p = rem / g.Q;
            q = rem - p * g.Q;
        }
        const int h0 = p * g.stride - g.pad, w0 = q * g.stride - g.pad;
        const f16* xn = x + n * g.H * g.W * g.C_in;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            int ih = h0 + tr[s], iw = w0 + ts[s];
            bool ok = mok && tok[s] && (unsigned)ih < (unsigned)g.H && (unsigned)iw < (unsigned)g.W;
            xf[s] = ok ? *(const half8_t*)(xn + (ih * g.W + iw) * g.C_in + tc[s]) : zero8;
        }
    };

    f16* tl = &tile[wave][0];
    // XDMA: instruction h (0, 1) moves pixels 8h..8h+7 of a block, each pixel's
    // 64 k = one 128-byte line, lane l -> pixel 8h + l/8, piece (l%8) ^ swz,
    // slot l%8, with swz = ((8h + l/8) >> 1) & 7 (conflict-free fragment reads).
    const unsigned xbytes = (unsigned)g.N * g.H * g.W * g.C_in * 2u;
    const u32x4_t xrs = raw_buffer_rsrc(x, xbytes);
    auto fetch_dma = [&](int blk, int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int px = 8 * h + (lane >> 3);
            const int piece = (lane & 7) ^ (px >> 1);
            const int m = blk * 16 + px;
            unsigned off = 0x80000000u;
            if (blk < nblocks && m < g.M && piece * 8 < g.K) {
                // 1x1 stride-1 unpadded geometry only (checked by the launcher):
                // pixel m's K = C_in values are contiguous at m * C_in.
                off = (unsigned)((m * g.C_in + piece * 8) * 2);
            }
            const unsigned la = (unsigned)(uintptr_t)(
                (__attribute__((address_space(3))) f16*)&xst[XDMA ? wave : 0][buf][h * 512]);
            lds_dma16(xrs, off, __builtin_amdgcn_readfirstlane(la));
        }
    };
    const int ocs = (lane % LPRW) * 8;        // channel within the slice, store phase
    const int orow = lane / LPRW;             // first tile row, store phase
    const bool vec_store = (g.C_out & 7) == 0;
    half8_t xc[KS], xn_[KS];
    int blk = stream;
    if (XDMA) {
#pragma unroll
        for (int d = 0; d < PD; ++d) fetch_dma(blk + d * nstreams, d);
    } else {
        fetch(blk, xc);
    }
    for (int it = 0; blk < nblocks; blk += nstreams, ++it) {
        const int B = it % PD;
        if (XDMA) {
            // Wait for this block's two direct-to-LDS loads only, not for the
            // stores issued after them. Every iteration issues exactly two
            // loads (after its MFMAs) and two stores (C_out % CW == 0 and a
            // full block; only a wave's last block may be partial), so the
            // loads of block it are followed by 2*(PD-1-it) + 4*it operations
            // when it < PD (prologue fetch) and by 2 + 4*(PD-1) afterwards.
            if (it < PD) wait_vmcnt<2 * (PD - 1)>(); else wait_vmcnt<4 * PD - 2>();
            const f16* xb = &xst[wave][B][0];
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int pc = 4 * s + lg;
                xc[s] = *(const half8_t*)(xb + lr * 64 + ((pc ^ (lr >> 1)) & 7) * 8);
            }
        }
        float4_t acc[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[f] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int f = 0; f < NF; ++f)
                acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[f][s], xc[s], acc[f], 0, 0, 0);
        if (XDMA) fetch_dma(blk + PD * nstreams, B);
        else fetch(blk + nstreams, xn_);  // after the MFMAs have consumed xc
#pragma unroll
        for (int j = 0; j < NF / 2; ++j) {
            half8_t h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h[e] = (f16)epilogue<EPI>(acc[2 * j][e], sc[j][e], bi[j][e]);
                h[4 + e] = (f16)epilogue<EPI>(acc[2 * j + 1][e], sc[j][4 + e], bi[j][4 + e]);
            }
            *(half8_t*)(tl + lr * TROW + 32 * j + 8 * lg) = h;
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < 16 / RPS; ++i) {
            const int row = orow + RPS * i;
            const int m = blk * 16 + row;
            const half8_t v = *(const half8_t*)(tl + row * TROW + ocs);
            const int o = c0 + ocs;
            if (m < g.M && o < g.C_out) {
                if (vec_store) {
                    store_y8<NT>(y, m * g.C_out + o, v, g.out8, g.res);
                } else {
                    for (int e = 0; e < 8; ++e)
                        if (o + e < g.C_out) store_y1(y, m * g.C_out + o + e, v[e], g.out8, g.res);
                }
            }
        }
        wave_lds_sync();
        if (!XDMA) {
#pragma unroll
            for (int s = 0; s < KS; ++s) xc[s] = xn_[s];
        }
    }
}

hipError_t launch_igemm_stream(const ConvGeom& g, int waves_per_cu, int xdma, bool nt, int epi,
                               const void* x, const void* w, const float* scale,
                               const float* bias, void* y, hipStream_t s) {
    const int NF = 4, CW = 64;
    int ngroups = (g.C_out + CW - 1) / CW;
    int nblocks = (g.M + 15) / 16;
    // grid*4 waves, a multiple of ngroups, about waves_per_cu per CU, at most
    // one wavefront per (block, group).
    long long want = 256LL * waves_per_cu;
    long long cap = (long long)nblocks * ngroups;
    if (want > cap) want = cap;
    long long waves = (want + ngroups - 1) / ngroups * ngroups;
    // round up to a multiple of 4 * ngroups / gcd -> simplest: multiple of 4*ngroups
    waves = (waves + 4LL * ngroups - 1) / (4LL * ngroups) * (4LL * ngroups);
    int grid = (int)(waves / 4);
    int ks = g.K <= 32 ? 1 : 2;
    const bool xdma_ok = g.kh == 1 && g.kw == 1 && g.stride == 1 && g.pad == 0 && ks == 2 &&
                         g.C_in == 64 && g.C_out % CW == 0;
    // xdma = d (1..4) selects the full-line staging path with prefetch depth d.
    int pd = xdma_ok ? xdma : 0;
    if (pd < 0 || pd > 4) pd = 0;
#define TG_ST_LAUNCH(KSV, EPI, NTV)                                                              \
    do {                                                                                         \
        switch (pd) {                                                                            \
            case 1: TG_ST_KERNEL(KSV, EPI, NTV, true, 1); break;                                \
            case 2: TG_ST_KERNEL(KSV, EPI, NTV, true, 2); break;                                \
            case 3: TG_ST_KERNEL(KSV, EPI, NTV, true, 3); break;                                \
            case 4: TG_ST_KERNEL(KSV, EPI, NTV, true, 4); break;                                \
            default: TG_ST_KERNEL(KSV, EPI, NTV, false, 1); break;                              \
        }                                                                                        \
    } while (0)
#define TG_ST_KERNEL(KSV, EPI, NTV, XD, PDV)                                                     \
    hipLaunchKernelGGL((conv2d_bn_silu_igemm_stream<NF, KSV, EPI, NTV, XD, PDV>), dim3(grid),    \
                       dim3(256), 0, s, (const f16*)x, (const f16*)w, scale, bias, (f16*)y, g,   \
                       nblocks, ngroups)
    // (tuning variant: BatchNorm+SiLU and identity epilogues only)
    if (epi != EPI_FUSED && epi != EPI_IDENTITY) return hipErrorInvalidValue;
    const bool identity = epi == EPI_IDENTITY;
    if (ks == 1) {
        if (identity) { if (nt) TG_ST_LAUNCH(1, EPI_IDENTITY, true); else TG_ST_LAUNCH(1, EPI_IDENTITY, false); }
        else { if (nt) TG_ST_LAUNCH(1, EPI_FUSED, true); else TG_ST_LAUNCH(1, EPI_FUSED, false); }
    } else {
        if (identity) { if (nt) TG_ST_LAUNCH(2, EPI_IDENTITY, true); else TG_ST_LAUNCH(2, EPI_IDENTITY, false); }
        else { if (nt) TG_ST_LAUNCH(2, EPI_FUSED, true); else TG_ST_LAUNCH(2, EPI_FUSED, false); }
    }
#undef TG_ST_KERNEL
#undef TG_ST_LAUNCH
    return hipGetLastError();
}

bool igemm_rw_serves(const ConvGeom& g) {
    long long xbytes = 2LL * g.N * g.H * g.W * g.C_in;
    return g.C_in % 8 == 0 && g.K <= 64 && g.C_out <= 256 && xbytes < (1LL << 31);
}

// Variants (NF, KS, CSPLIT, NCW).
#define TG_RW_CFGS(X)                                                                \
    X(4, 1, 1, 4) X(4, 2, 1, 4) X(4, 1, 2, 4) X(4, 2, 2, 4) X(4, 1, 4, 8) X(4, 2, 4, 8) \
    X(8, 1, 2, 4) X(8, 2, 2, 4) X(4, 2, 4, 4) X(4, 2, 2, 8)

bool igemm_rw_valid(const ConvGeom& g, int nf, int cs, int ncw) {
    const int ks = g.K <= 32 ? 1 : 2;
    if (nf * 16 * cs < g.C_out) return false;
#define X(NF_, KS_, CS_, NCW_) \
    if (nf == NF_ && ks == KS_ && cs == CS_ && ncw == NCW_) return true;
    TG_RW_CFGS(X)
#undef X
    return false;
}

void igemm_rw_choose(const ConvGeom& g, int* nf, int* cs, int* ncw) {
    if (g.C_out <= 64) { *nf = 4; *cs = 1; *ncw = 4; }
    else if (g.C_out <= 128) { *nf = 4; *cs = 2; *ncw = 4; }
    else { *nf = 4; *cs = 4; *ncw = 8; }
}

// Persistent grid: at most `slots` workgroups, at least one 16-pixel block
// per round slot.
int igemm_rw_grid(const ConvGeom& g, int slots) {
    int nblocks = (g.M + 15) / 16;
    int grid = (nblocks + 1) / 2;
    return grid < slots ? grid : slots;
}

template <int NF, int KS, int CS, int NCW>
static void launch_rw_one(const ConvGeom& g, int grid, int epi, bool nt, const void* x,
                          const void* w, const float* scale, const float* bias, void* y,
                          hipStream_t s) {
    int nblocks = (g.M + 15) / 16;
#define TG_RW_LAUNCH(EPI, NTV)                                                              \
    hipLaunchKernelGGL((conv2d_bn_silu_igemm_rw<NF, KS, CS, NCW, EPI, NTV>), dim3(grid),     \
                       dim3((NCW + 1) * 64), 0, s, (const f16*)x, (const f16*)w, scale, bias, \
                       (f16*)y, g, nblocks)
#define TG_RW_NT(E)                \
    do {                           \
        if (nt) TG_RW_LAUNCH(E, true); \
        else TG_RW_LAUNCH(E, false);   \
    } while (0)
    TG_EPI_DISPATCH(epi, TG_RW_NT);
#undef TG_RW_NT
#undef TG_RW_LAUNCH
}

hipError_t launch_igemm_rw(const ConvGeom& g, int grid, int nf, int cs, int ncw, bool nt,
                           int epi, const void* x, const void* w, const float* scale,
                           const float* bias, void* y, hipStream_t s) {
    int ks = g.K <= 32 ? 1 : 2;
    if (nf * 16 * cs < g.C_out) return hipErrorInvalidValue;
#define X(NF_, KS_, CS_, NCW_)                                                               \
    if (nf == NF_ && ks == KS_ && cs == CS_ && ncw == NCW_) {                                \
        launch_rw_one<NF_, KS_, CS_, NCW_>(g, grid, epi, nt, x, w, scale, bias, y, s);     \
        return hipGetLastError();                                                            \
    }
    TG_RW_CFGS(X)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace tg
