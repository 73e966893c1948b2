// igemm_patch.hip -- conv2d_bn_silu_igemm for stride-1 convolutions with
// C_in % 64 == 0 (the 3x3 and 7x7 layers): the input patch of a tile is
// staged in LDS once and serves every filter tap.
//
// Same operation as igemm.hip ("Fusing an Epilogue", teenygrad docs, "The
// shape of it": the K-loop on the matrix cores leaves the output tile in
// registers, BatchNorm scale/shift and SiLU are applied there, then one
// store). The implicit-GEMM formulation reads an input pixel once per filter
// tap (9 or 49 times); here a workgroup's tile is BM consecutive output
// pixels of one image, and the input rows they touch -- all C_in channels,
// zero-padded at the image border -- are copied into LDS once:
//   * the rows filter row 0 needs are copied by all compute waves before
//     the K loop; each later filter row needs one more patch row, which a
//     loader wave streams in with direct-to-LDS loads while the K loop runs
//     and publishes through an LDS flag (at kernel start every workgroup
//     wants its whole patch at once, so the copy was HBM-bound time with the
//     matrix cores idle);
//   * patch pixel stride is C_in*2 + 32 bytes (2 mod 4 16-byte units), which
//     measured conflict-free on gfx950 for 16 consecutive pixels read at one
//     channel piece -- no swizzle that would depend on the tap's shift (the
//     denser C_in*2 + 16 costs 2-way conflicts and is the fallback when LDS
//     is short). When LDS allows, patch rows are padded to Q + 16 pixels: a
//     fragment whose 16 pixels wrap to the next output row then jumps by 16
//     pixels, which keeps the same bank groups;
//   * for tap (r, s) a lane's fragment address is its tap-(0,0) address plus
//     a wave-uniform (r*PW + s)*stride: one add per fragment and tap;
//   * only the filter chunks stream (64 channels of one tap). Each wave
//     fetches the rows and the half (or whole) 128-byte chunk row its own
//     fragments need into a wave-private 3- or 4-stage ring with direct-to-LDS
//     loads (rows XOR-swizzled), so the main loop has no workgroup barrier:
//     a wave waits only for its own loads, with an exact vmcnt; per-lane
//     offsets are precomputed so that a chunk costs one add per load;
//   * WK = 2 runs two groups of four waves on the two 32-deep halves of every
//     chunk (two waves per SIMD: one's fragment reads overlap the other's
//     MFMAs); their partial tiles are summed through LDS before the epilogue,
//     so the epilogue sees the complete K sum.
//
// Load-time filter pre-pack ("When the fusion you want is impossible, fuse
// into the producer", section "The general form": work repeated at every call
// that could be done once at load time belongs at load time; there the
// channels-last filters left the output bit-identical): pack_patch_filter rewrites
// the OHWI filter into the order in which this kernel's direct-to-LDS loads
// land in its filter ring -- per 64-channel chunk kc, per block of 16 output
// channels ob, per K-group kg, 16 rows of 128/WK bytes whose 16-byte pieces
// are already XOR-swizzled -- so that every filter load instruction of a
// wave reads one contiguous kilobyte instead of 16 (or 8) row fragments:
//   byte ((kc*NB + ob)*WK + kg)*(2048/WK) + rr*(128/WK) + s*16 holds
//   w[16*ob + rr][64*kc + kg*(64/WK) + 8*(s ^ swz(rr)) .. + 7]
// (NB = ceil(C_out/16); rows past C_out are zero; swz is pt_wswz<WK>). The
// kernel's LDS contents, and therefore its arithmetic, are the same for both
// forms.
#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {
namespace {

__device__ __forceinline__ void pt_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void pt_wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ u32x4_t pt_rsrc(const void* base, unsigned bytes) {
    const unsigned long long a = (unsigned long long)base;
    u32x4_t r;
    r[0] = (unsigned)a;
    r[1] = (unsigned)(a >> 32) & 0xffffu;
    r[2] = bytes;
    r[3] = 0x00020000u;
    return r;
}

// 16-byte direct-to-LDS load (lane l -> lds + 16*l; offsets past num_records
// read zeros); ordered by the caller's explicit vmcnt waits.
__device__ __forceinline__ void pt_dma16(u32x4_t rsrc, unsigned voff, unsigned lds) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds)
                 : "memory");
}

// 16-byte LDS read issued as inline asm: the compiler does not track it, so
// its completion is the caller's explicit lgkmcnt wait (pt_frag_wait). The
// compiler's own tracking turned conservative in this kernel's K loop and
// waited for the next chunk's fragment reads before the current chunk's
// MFMAs, which serialised LDS and the matrix cores.
__device__ __forceinline__ half8_t pt_lds16(unsigned addr) {
    half8_t r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr) : "memory");
    return r;
}

// s_waitcnt lgkmcnt(n) for a count known after unrolling (the counter field
// holds 0..15; larger counts wait for 15, which is stricter).
__device__ __forceinline__ void pt_wait_lgkm(int n) {
    switch (n < 15 ? n : 15) {
#define TG_LGKM(N)                                              \
    case N:                                                     \
        asm volatile("s_waitcnt lgkmcnt(" #N ")" ::: "memory"); \
        break;
        TG_LGKM(0) TG_LGKM(1) TG_LGKM(2) TG_LGKM(3) TG_LGKM(4) TG_LGKM(5) TG_LGKM(6) TG_LGKM(7)
        TG_LGKM(8) TG_LGKM(9) TG_LGKM(10) TG_LGKM(11) TG_LGKM(12) TG_LGKM(13) TG_LGKM(14)
        TG_LGKM(15)
#undef TG_LGKM
    }
}

// Fragment reads of one step are issued in order r = 0..NL-1 (per 32-deep
// half kk: FN filter fragments, then FM pixel fragments); MFMA m reads
// filter fragment (kk, i) and pixel fragment (kk, j). The highest read index
// any of MFMAs 0..m uses:
template <int FN, int FM>
__host__ __device__ constexpr int pt_reads_needed(int m) {
    int hi = 0;
    for (int k = 0; k <= m; ++k) {
        const int kk = k / (FN * FM), i = (k / FM) % FN, j = k % FM;
        const int ra = kk * (FN + FM) + i, rb = kk * (FN + FM) + FN + j;
        hi = hi > ra ? hi : ra;
        hi = hi > rb ? hi : rb;
    }
    return hi;
}

template <int BM, int BN, int WM, int WN, int WK, int RING>
struct PatchShape {
    static_assert(RING == 3 || RING == 4, "filter ring of three or four stages");
    static constexpr int WPG = WM * WN;                // waves per K-group
    static_assert(WPG == 2 || WPG == 4, "two or four waves per K-group");
    static_assert(WK == 1 || WK == 2, "one or two K-groups");
    static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tiles of 16x16 blocks");
    static constexpr int NW = WPG * WK;
    static constexpr int FM = BM / WM / 16, FN = BN / WN / 16;
    static constexpr int PPR = 8 / WK;                 // 16-byte pieces of a wave's chunk row
    static constexpr int LI = FN * 16 * PPR / 64;      // filter loads per chunk per wave
    static_assert(FN * 16 * PPR % 64 == 0, "whole load instructions");
    static constexpr int WSTAGE = FN * 16 * PPR * 16;  // bytes per stage of a wave's ring
    static constexpr int RING_BYTES = NW * RING * WSTAGE;
    static constexpr int OROW = BN + 8;                // output tile row (halves)
    static constexpr int RED_BYTES = WK == 2 ? WPG * FN * FM * 64 * 16 : 0;
    static constexpr int EPI_BYTES = RED_BYTES + BM * OROW * 2;
    static_assert(LI * RING <= 63, "vmcnt range");
};

// Slot of piece p in row r of a wave's filter stage is p ^ pt_wswz<WK>(r):
// (r/2)%4 for 64-byte rows (WK = 2) and (r/2)%8 for 128-byte rows; both
// measured conflict-free on gfx950 for 16 rows x one piece per lane group.
template <int WK>
__device__ __forceinline__ int pt_wswz(int r) {
    return WK == 2 ? (r >> 1) & 3 : (r >> 1) & 7;
}

template <int BM, int BN, int WM, int WN, int WK, int RING, int EPI>
__global__ __launch_bounds__(64 * (WM * WN * WK + 1), 1) void conv2d_bn_silu_igemm_patch(
    const f16* __restrict__ x, const f16* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, f16* __restrict__ y, ConvGeom g, int tiles_per_img,
    int tiles_n, int PW, int pstride, int packed) {
    using S = PatchShape<BM, BN, WM, WN, WK, RING>;
    extern __shared__ __attribute__((aligned(16))) unsigned char pt_smem[];

    const int tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    const int tn = tile % tiles_n, tmi = tile / tiles_n;
    const int n = tmi / tiles_per_img, t = tmi - n * tiles_per_img;
    const int PQ = g.P * g.Q;
    const int r0 = t * BM;                              // first output pixel in the image
    const int r1 = r0 + BM < PQ ? r0 + BM : PQ;         // one past the last valid one
    const int p_first = r0 / g.Q, p_last = (r1 - 1) / g.Q;
    const int PR = p_last - p_first + g.kh;             // patch rows
    // PW: patch columns, Q + kw - 1 or (padded) Q + 16; columns past
    // Q + kw - 2 are never read. pstride: bytes per patch pixel, C_in*2 + 32
    // (conflict-free) or, when that does not fit, C_in*2 + 16.
    const int n0 = tn * BN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = wave / S::WPG, w4 = wave - kg * S::WPG;  // K-group, wave within it
    const int wm = w4 / WN, wn = w4 - (w4 / WN) * WN;
    const int lr = lane & 15, lg = lane >> 4;
    const int cchunks = g.C_in / 64;
    const int nk = g.kh * g.kw * cchunks;

    // LDS: [patch-progress flag (16 B)][rings][patch]; the epilogue reuses
    // all of it once the K loop is done.
    int* pflag = (int*)pt_smem;  // filter rows whose patch rows have landed
    unsigned char* ring = pt_smem + 16 + wave * RING * S::WSTAGE;  // this wave's ring
    unsigned char* patch = pt_smem + 16 + S::RING_BYTES;
    const unsigned patch_lds = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)patch));
    // Compute waves: patch rows of filter row r are in LDS once the flag
    // exceeds r.
    auto wait_rows = [&](int r) {
        while (__hip_atomic_load(pflag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) <= r)
            __builtin_amdgcn_s_sleep(1);
        asm volatile("" ::: "memory");
    };
    const unsigned ring_lds = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)ring));

    // Filter chunk loads: this wave needs rows wn*FN*16 .. +FN*16 of the
    // BN-row tile and pieces kg*PPR .. +PPR of each 128-byte chunk row.
    // Instruction i moves 64/PPR rows; lane l takes row i*64/PPR + l/PPR,
    // piece (l%PPR) ^ pt_wswz(row) -> slot l%PPR. From a packed filter the
    // same bytes are lane l's 16 bytes of one contiguous kilobyte.
    const int NB = (g.C_out + 15) / 16;
    const unsigned kstride = packed ? (unsigned)NB * 2048u : 128u;  // bytes per chunk
    const u32x4_t wrs = pt_rsrc(w, packed ? (unsigned)nk * kstride
                                          : (unsigned)g.C_out * (unsigned)g.K * 2u);
    unsigned woff[S::LI];
#pragma unroll
    for (int i = 0; i < S::LI; ++i) {
        const int rb = i * (64 / S::PPR);  // first wave-local row of instruction i
        if (packed) {
            const int ob = (n0 + wn * S::FN * 16 + rb) / 16;
            woff[i] = ob < NB ? (unsigned)((ob * WK + (WK == 2 ? kg : 0)) * (2048 / WK) +
                                           (rb % 16) * (128 / WK) + 16 * lane)
                              : 0x80000000u;
        } else {
            const int row = rb + lane / S::PPR;
            const int piece = (lane % S::PPR) ^ pt_wswz<WK>(row);
            const int o = n0 + wn * S::FN * 16 + row;
            const int kp = (WK == 2 ? kg * S::PPR : 0) + piece;
            woff[i] = o < g.C_out ? (unsigned)((o * g.K + kp * 8) * 2) : 0x80000000u;
        }
    }
    // Chunk kc's filter loads; past the last chunk they read zeros (out of
    // the buffer's range) so that every step issues the same loads.
    auto issue = [&](int kc) {
        // Chunk kc is K range [64 kc, 64 kc + 64) (tap kc / cchunks, channel
        // chunk kc % cchunks, since C_in = 64 cchunks): 128 bytes of each
        // OHWI row, or one packed slab of NB * 2048 bytes.
        const unsigned koff = kc < nk ? (unsigned)kc * kstride : 0x80000000u;
        const unsigned dst = ring_lds + (unsigned)(kc % RING) * S::WSTAGE;
#pragma unroll
        for (int i = 0; i < S::LI; ++i) pt_dma16(wrs, woff[i] + koff, dst + i * 1024);
    };
    if (wave < S::NW)
        for (int kc = 0; kc < RING - 1; ++kc) issue(kc);

    const int orows = p_last - p_first + 1;  // output rows of the tile

    // Patch rows [0, orows) -- all that filter row 0 needs -- copied by the
    // compute waves together: PR x PW pixels x C_in channels, zeros outside
    // the image. Thread u copies 16-byte piece (u % upp) of pixels u/upp,
    // u/upp + step, ... (64*NW is a multiple of upp = C_in/8, so the piece
    // is fixed).
    if (wave < S::NW) {
        const int upp = g.C_in / 8;
        const int npx = orows * PW;
        const int step = 64 * S::NW / upp;
        const int piece = threadIdx.x % upp;
        int px = threadIdx.x / upp;
        int pr = px / PW, pc = px - (px / PW) * PW;
        const int step_r = step / PW, step_c = step - step_r * PW;
        const f16* xn = x + (size_t)n * g.H * g.W * g.C_in + piece * 8;
        const half8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
        constexpr int B = 8;  // loads in flight per thread
        while (px < npx) {
            half8_t v[B];
            int dst[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const int ih = p_first - g.pad + pr, iw = pc - g.pad;
                const bool ok = px < npx && (unsigned)ih < (unsigned)g.H &&
                                (unsigned)iw < (unsigned)g.W;
                v[b] = ok ? *(const half8_t*)(xn + (ih * g.W + iw) * g.C_in) : zero8;
                dst[b] = px < npx ? px * pstride + piece * 16 : -1;
                px += step;
                pr += step_r;
                pc += step_c;
                if (pc >= PW) { pc -= PW; ++pr; }
            }
#pragma unroll
            for (int b = 0; b < B; ++b)
                if (dst[b] >= 0) *(half8_t*)(patch + dst[b]) = v[b];
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(pflag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();  // filter row 0's patch rows are in LDS

    if (wave == S::NW) {
        // ---------------- patch loader wave ----------------
        // Filter row r (r >= 1) needs patch row orows + r - 1 as well: the
        // remaining rows stream in that order while the K loop runs, one
        // phase per filter row, each published once its loads have landed.
        // A load instruction fills PPI whole patch pixels: lane l takes
        // 16-byte piece l % PP of pixel l / PP (pieces past the C_in*2 data
        // bytes and pixels outside the image read zeros).
        const int PP = pstride / 16, PPI = 64 / PP;
        const int lp = lane / PP, piece = lane - lp * PP;
        const bool lane_on = lane < PPI * PP;
        const bool data = piece * 16 < g.C_in * 2;
        const u32x4_t xrs = pt_rsrc(x, (unsigned)g.N * (unsigned)g.H * (unsigned)g.W * (unsigned)g.C_in * 2u);
        int cur = orows * PW;  // first pixel of the next load instruction
        int pix = cur + lp, pr = pix / PW, pc = pix - (pix / PW) * PW;
        for (int r = 1; r < g.kh; ++r) {
            const int pend = (orows + r) * PW;
            for (; cur < pend; cur += PPI) {
                const int ih = p_first - g.pad + pr, iw = pc - g.pad;
                const bool ok = data && (unsigned)ih < (unsigned)g.H && (unsigned)iw < (unsigned)g.W;
                const unsigned off =
                    ok ? (unsigned)((((n * g.H + ih) * g.W + iw) * g.C_in + piece * 8) * 2) : 0x80000000u;
                if (lane_on && pix < PR * PW) pt_dma16(xrs, off, patch_lds + (unsigned)(cur * pstride));
                pix += PPI;
                pc += PPI;
                while (pc >= PW) {
                    pc -= PW;
                    ++pr;
                }
            }
            pt_wait_vmcnt<0>();
            __hip_atomic_store(pflag, r + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        return;
    }

    // Fragment addresses for tap (0, 0), channel piece lg: x operand (pixels)
    // from the patch, weight operand from the ring stage (ks = 1 is ks = 0
    // with slot bit 2 flipped, i.e. byte offset ^ 64).
    int abase[S::FM];
#pragma unroll
    for (int f = 0; f < S::FM; ++f) {
        int r = r0 + (wm * S::FM + f) * 16 + lr;
        if (r > r1 - 1) r = r1 - 1;  // beyond the tile: any valid pixel, result unused
        const int p = r / g.Q, q = r - (r / g.Q) * g.Q;
        abase[f] = ((p - p_first) * PW + q) * pstride + lg * 16;
    }
    int bbase[S::FN];  // piece lg (ks = 0) of row f*16 + lr; ks = 1 (WK = 1): ^ 64
#pragma unroll
    for (int f = 0; f < S::FN; ++f) {
        const int row = f * 16 + lr;
        bbase[f] = row * S::PPR * 16 + ((lg ^ pt_wswz<WK>(row)) * 16);
    }

    float4_t acc[S::FN][S::FM];
#pragma unroll
    for (int a = 0; a < S::FN; ++a)
#pragma unroll
        for (int b = 0; b < S::FM; ++b) acc[a][b] = (float4_t){0.f, 0.f, 0.f, 0.f};

    // Fragments of chunk kc for this wave's 32-deep step(s): registers are
    // double-buffered so that chunk kc+1's fragment reads overlap chunk kc's
    // MFMAs (software pipelining across chunks).
    constexpr int KSW = 2 / WK;  // 32-deep steps per chunk for this wave
    struct Frags {
        half8_t a[KSW][S::FN], b[KSW][S::FM];
    };
    // Wait for every outstanding fragment read, after the MFMAs that read
    // F: F's registers pass through (empty) volatile asm statements placed
    // before the wait, which orders those MFMAs ahead of it, so the wait
    // overlaps their execution.
    auto frag_wait = [&](Frags& F) {
#pragma unroll
        for (int kk = 0; kk < KSW; ++kk) {
#pragma unroll
            for (int f = 0; f < S::FN; ++f) asm volatile("" : "+v"(F.a[kk][f]));
#pragma unroll
            for (int f = 0; f < S::FM; ++f) asm volatile("" : "+v"(F.b[kk][f]));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };
    // Chunk kc's filter data has landed once only the loads of the RING - 2
    // chunks issued after it are pending (chunks run RING - 1 ahead).
    auto wait_chunk = [&]() { pt_wait_vmcnt<(RING - 2) * S::LI>(); };
    // MFMA m of a step (m = (kk*FN + i)*FM + j: acc[i][j] += a[kk][i] x
    // b[kk][j], the order of the plain triple loop) as inline assembly, so
    // that it keeps its place in program order between the step's filter
    // loads and LDS reads (also inline assembly). The compiler schedules a
    // builtin MFMA freely and put all of a step's MFMAs in one run after the
    // step's other instructions; the wave then issued those with the matrix
    // core idle, and on both waves of a SIMD at once.
    auto mfma = [&](const Frags& F, int m) {
        const int kk = m / (S::FN * S::FM), i = (m / S::FM) % S::FN, j = m % S::FM;
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                     : "+v"(acc[i][j])
                     : "v"(F.a[kk][i]), "v"(F.b[kk][j]));
    };
    // Read r of a chunk's fragments (kk = r / (FN + FM): FN filter
    // fragments from ring stage st, then FM pixel fragments at patch offset
    // delta).
    auto read = [&](Frags& F, int r, unsigned st, unsigned delta) {
        const int kk = r / (S::FN + S::FM), q = r % (S::FN + S::FM);
        const int ks = WK == 2 ? kg : kk;
        if (q < S::FN)
            F.a[kk][q] = pt_lds16(st + (unsigned)(bbase[q] ^ (WK == 2 ? 0 : ks * 64)));
        else
            F.b[kk][q - S::FN] = pt_lds16(patch_lds + (unsigned)(abase[q - S::FN] + ks * 64) + delta);
    };
    // (tap_r, tap_s, cc) of the chunk whose fragments are loaded next;
    // advanced with selects, not branches.
    int tap_r = 0, tap_s = 0, cc = 0;
    auto advance = [&]() {
        const bool wc = cc + 1 == cchunks;
        cc = wc ? 0 : cc + 1;
        const bool ws = wc && tap_s + 1 == g.kw;
        tap_s = ws ? 0 : (wc ? tap_s + 1 : tap_s);
        tap_r = ws ? tap_r + 1 : tap_r;
    };
    constexpr int NM = KSW * S::FN * S::FM;    // MFMAs per step
    constexpr int NL = KSW * (S::FN + S::FM);  // fragment reads per step
    Frags F0, F1;
    wait_chunk();
    wait_rows(0);
#pragma unroll
    for (int r = 0; r < NL; ++r) read(F0, r, ring_lds, 0u);
    advance();
    frag_wait(F0);
    // One step: refill the ring, fetch chunk kc+1's fragments into `nxt`,
    // run chunk kc's MFMAs from `cur`, then wait for the fetch (it overlaps
    // the MFMAs). Stage (kc + RING - 1) % RING was last read for chunk
    // kc - 1, whose fragment reads completed at the end of step kc - 2.
    // The step's other instructions sit between its MFMAs, one group after
    // each: the filter loads after the first, the ring wait (and at a
    // filter row's first chunk the patch-row wait) after the second, then
    // one fragment read after each further MFMA. The matrix core works
    // through the earlier MFMAs meanwhile.
    // The last step reads fragments too (one MFMA sequence in the code, not
    // two): at patch offset 0 and a ring stage that the trailing zero-filling
    // filter loads may be writing, values no MFMA uses. The fragment
    // registers are kept live past the LDS wait after the loop, so that no
    // other value is given a register a late LDS write would overwrite.
    // The fragments of `cur` were read during the previous step, and LDS
    // operations complete in order: MFMA m waits only for the reads it uses
    // (all but NL - 1 - pt_reads_needed(m) of them, plus the reads of `nxt`
    // issued in this step before it), so the step's first MFMAs overlap the
    // latency of its last fragment reads.
    // Each fragment then passes through an empty asm statement that claims
    // to modify it, right after the wait that completes its read: no copy
    // or use of the register can be placed before that wait.
    auto frag_ready = [&](Frags& F, int m) {
        const int need = pt_reads_needed<S::FN, S::FM>(m);
        const int prev = m == 0 ? -1 : pt_reads_needed<S::FN, S::FM>(m - 1);
        if (need > prev) {
            const int issued = m < 2 ? 0 : (m - 2 < NL ? m - 2 : NL);
            pt_wait_lgkm(NL - 1 - need + issued);
#pragma unroll
            for (int r = 0; r < NL; ++r) {
                if (r <= prev || r > need) continue;
                const int kk = r / (S::FN + S::FM), q = r % (S::FN + S::FM);
                if (q < S::FN)
                    asm volatile("" : "+v"(F.a[kk][q]));
                else
                    asm volatile("" : "+v"(F.b[kk][q - S::FN]));
            }
        }
    };
    auto step = [&](int kc, Frags& cur, Frags& nxt) {
        const bool more = kc + 1 < nk;
        const bool row_wait = more && tap_s == 0 && cc == 0;  // first chunk of a filter row
        const unsigned st = ring_lds + (unsigned)(((kc + 1) % RING) * S::WSTAGE);
        const unsigned delta = more ? (unsigned)((tap_r * PW + tap_s) * pstride + cc * 128) : 0u;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            frag_ready(cur, m);
            mfma(cur, m);
            if (m == 0) issue(kc + RING - 1);
            if (m == 1) {
                wait_chunk();
                if (row_wait) wait_rows(tap_r);
            }
            if (m >= 2 && m - 2 < NL) read(nxt, m - 2, st, delta);
        }
#pragma unroll
        for (int r = NM - 2; r < NL; ++r) read(nxt, r > 0 ? r : 0, st, delta);
        advance();
    };
    // Pairs of steps in straight-line code (the compiler's wait counts stay
    // exact across the back edge), then an odd last step.
    int kc = 0;
    for (; kc + 1 < nk; kc += 2) {
        step(kc, F0, F1);
        step(kc + 1, F1, F0);
    }
    if (kc < nk) {  // odd last step: nothing left to fetch
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(kc + RING - 1);
#pragma unroll
        for (int m = 0; m < NM; ++m) mfma(F0, m);
    }
    // The last step's fragment reads (values no MFMA uses) land before
    // their registers are released.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int kk = 0; kk < KSW; ++kk) {
#pragma unroll
        for (int f = 0; f < S::FN; ++f) asm volatile("" ::"v"(F0.a[kk][f]), "v"(F1.a[kk][f]));
#pragma unroll
        for (int f = 0; f < S::FM; ++f) asm volatile("" ::"v"(F0.b[kk][f]), "v"(F1.b[kk][f]));
    }
    // The accumulators are read below by LDS stores and VALU: the matrix
    // core's last results must be written first (inline-assembly MFMAs get
    // no hazard padding from the compiler; 32 wait states cover the
    // 8-pass 16x16x32 MFMA with margin).
    asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
    // The last steps' filter loads (past the last chunk, zero-filling) land
    // in the ring asynchronously: drain them before the ring's LDS is reused.
    pt_wait_vmcnt<0>();
    pt_barrier();  // every wave is done with its ring and the patch: reuse LDS

    // WK = 2: the two K-groups share the epilogue. Group 0 owns fragment
    // columns j < JH, group 1 the rest; each hands its partial sums of the
    // other group's fragments over through LDS and adds the ones it gets.
    constexpr int JH = (S::FM + 1) / 2;
    auto owned = [&](int j) { return WK == 1 || (j < JH) == (kg == 0); };
    if (WK == 2) {
        float4_t* red = (float4_t*)pt_smem + w4 * S::FN * S::FM * 64 + lane;
#pragma unroll
        for (int i = 0; i < S::FN; ++i)
#pragma unroll
            for (int j = 0; j < S::FM; ++j)
                if (!owned(j)) red[(i * S::FM + j) * 64] = acc[i][j];
        pt_barrier();
#pragma unroll
        for (int i = 0; i < S::FN; ++i)
#pragma unroll
            for (int j = 0; j < S::FM; ++j)
                if (owned(j)) acc[i][j] += red[(i * S::FM + j) * 64];
    }

    {
        // Lane holds channels cb..cb+3 of tile pixel pr for each block.
        f16* out = (f16*)(pt_smem + S::RED_BYTES);
#pragma unroll
        for (int i = 0; i < S::FN; ++i) {
            const int cb = wn * S::FN * 16 + i * 16 + lg * 4;
            float sc[4], bi[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) epi_consts<EPI>(scale, bias, n0 + cb + e, g.C_out, sc[e], bi[e]);
#pragma unroll
            for (int j = 0; j < S::FM; ++j) {
                if (!owned(j)) continue;
                const int pr = wm * S::FM * 16 + j * 16 + lr;
                half4_t h;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    h[e] = (f16)epilogue<EPI>(acc[i][j][e], sc[e], bi[e]);
                *(half4_t*)(out + pr * S::OROW + cb) = h;
            }
        }
    }

    // y leaves with non-temporal stores: nothing in this kernel reads it
    // again (measured on the 3x3 and 7x7 layers: ~3% faster than plain).
    pt_barrier();
    {
        const f16* out = (const f16*)(pt_smem + S::RED_BYTES);
        const int rows = r1 - r0;
        constexpr int CV = BN / 8;
        if ((g.C_out & 7) == 0) {
            for (int v = threadIdx.x; v < BM * CV; v += 64 * S::NW) {
                const int row = v / CV, cv = v - (v / CV) * CV;
                const int o = n0 + cv * 8;
                if (row < rows && o < g.C_out)
                    store_y8<true>(y, ((long long)n * PQ + r0 + row) * g.C_out + o,
                             *(const half8_t*)(out + row * S::OROW + cv * 8), g.out8, g.res);
            }
        } else {
            for (int v = threadIdx.x; v < BM * BN; v += 64 * S::NW) {
                const int row = v / BN, c = v - (v / BN) * BN;
                const int o = n0 + c;
                if (row < rows && o < g.C_out)
                    store_y1(y, ((long long)n * PQ + r0 + row) * g.C_out + o, out[row * S::OROW + c],
                             g.out8, g.res);
            }
        }
    }
}

// BM, BN, WM, WN, WK, filter ring stages. The three-stage ring leaves room
// for the conflict-free patch stride where four stages would not.
#define TG_PATCH_CFGS(X)        \
    X(112, 128, 1, 2, 2, 4)     \
    X(224, 64, 2, 1, 2, 4)      \
    X(112, 128, 1, 4, 2, 4)     \
    X(224, 64, 2, 2, 2, 4)      \
    X(128, 64, 2, 2, 2, 4)      \
    X(64, 64, 2, 2, 2, 4)       \
    X(112, 128, 1, 4, 1, 4)     \
    X(224, 64, 2, 2, 1, 4)      \
    X(224, 64, 2, 2, 2, 3)      \
    X(112, 128, 1, 4, 2, 3)

struct PatchCfg {
    int BM, BN, WM, WN, WK, RING;
};
const PatchCfg kPatchCfgs[] = {
#define X(bm, bn, wm, wn, wk, ring) {bm, bn, wm, wn, wk, ring},
    TG_PATCH_CFGS(X)
#undef X
};
constexpr int kNumPatchCfgs = (int)(sizeof(kPatchCfgs) / sizeof(kPatchCfgs[0]));

// Rows of output pixels a BM-pixel tile can touch (tiles start at multiples
// of BM within an image).
int patch_rows_max(const ConvGeom& g, int BM) {
    const int PQ = g.P * g.Q;
    int worst = 0;
    for (int r0 = 0; r0 < PQ; r0 += BM) {  // exact over the tiles of one image
        const int r1 = r0 + BM < PQ ? r0 + BM : PQ;
        const int rows = (r1 - 1) / g.Q - r0 / g.Q + 1;
        if (rows > worst) worst = rows;
    }
    return worst;
}

size_t patch_lds_bytes_w(const ConvGeom& g, const PatchCfg& c, int pw, int pstride) {
    // Wave-private rings: WM*WN*WK waves x RING stages x (BN/WN rows x 128/WK bytes).
    const size_t ring = (size_t)c.WM * c.WN * c.WK * c.RING * (c.BN / c.WN) * (128 / c.WK);
    const size_t pr = (size_t)patch_rows_max(g, c.BM) + g.kh - 1;
    const size_t patch = pr * (size_t)pw * (size_t)pstride + 16;  // + progress flag
    const size_t red =
        c.WK == 2 ? (size_t)c.WM * c.WN * (c.BN / c.WN / 16) * (c.BM / c.WM / 16) * 64 * 16 : 0;
    const size_t epi = red + (size_t)c.BM * (c.BN + 8) * 2;
    return ring + patch > epi ? ring + patch : epi;
}

// Patch layout, best first: padded rows with the conflict-free stride, plain
// rows with it, plain rows with the dense stride.
struct PatchLayout {
    int pw, pstride;
};
PatchLayout patch_layout(const ConvGeom& g, const PatchCfg& c) {
    const int plain = g.Q + g.kw - 1, padded = g.Q + 16;
    const int wide = g.C_in * 2 + 32, dense = g.C_in * 2 + 16;
    if (g.kw <= 17 && padded > plain && patch_lds_bytes_w(g, c, padded, wide) <= 160 * 1024)
        return {padded, wide};
    if (patch_lds_bytes_w(g, c, plain, wide) <= 160 * 1024) return {plain, wide};
    return {plain, dense};
}

size_t patch_lds_bytes(const ConvGeom& g, const PatchCfg& c) {
    const PatchLayout L = patch_layout(g, c);
    return patch_lds_bytes_w(g, c, L.pw, L.pstride);
}

template <int BM, int BN, int WM, int WN, int WK, int RING>
hipError_t patch_launch_one(const ConvGeom& g, int epi, const void* x, const void* w,
                            const float* scale, const float* bias, void* y, bool packed,
                            hipStream_t s) {
    using S = PatchShape<BM, BN, WM, WN, WK, RING>;
    const PatchCfg c = {BM, BN, WM, WN, WK, RING};
    const size_t lds = patch_lds_bytes(g, c);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    const int tiles_per_img = (g.P * g.Q + BM - 1) / BM, tiles_n = (g.C_out + BN - 1) / BN;
    if (epi < 0 || epi >= kNumEpilogues) return hipErrorInvalidValue;
    auto k = conv2d_bn_silu_igemm_patch<BM, BN, WM, WN, WK, RING, EPI_FUSED>;
#define TG_K(E) k = conv2d_bn_silu_igemm_patch<BM, BN, WM, WN, WK, RING, E>
    TG_EPI_DISPATCH(epi, TG_K);
#undef TG_K
    hipError_t e = ensure_dynamic_lds((const void*)k, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(g.N * tiles_per_img * tiles_n), dim3(64 * (S::NW + 1)), lds, s,
                       (const f16*)x, (const f16*)w, scale, bias, (f16*)y, g, tiles_per_img,
                       tiles_n, patch_layout(g, c).pw, patch_layout(g, c).pstride,
                       packed ? 1 : 0);
    return hipGetLastError();
}

// One thread per 16-byte piece of the packed filter (layout in the header
// comment); WK = 1 or 2.
__global__ __launch_bounds__(256) void pack_patch_filter(const f16* __restrict__ w,
                                                         f16* __restrict__ wp, int C_out, int K,
                                                         int NB, int WK, long long npieces) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= npieces) return;
    const int ppr = 8 / WK;
    long long t = i / ppr;
    const int sl = (int)(i - t * ppr);
    const int rr = (int)(t % 16);
    t /= 16;
    const int kg = (int)(t % WK);
    t /= WK;
    const int ob = (int)(t % NB);
    const long long kc = t / NB;
    const int piece = sl ^ (WK == 2 ? pt_wswz<2>(rr) : pt_wswz<1>(rr));
    const int o = ob * 16 + rr;
    const long long k = kc * 64 + kg * (64 / WK) + 8 * piece;
    half8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (o < C_out) v = *(const half8_t*)(w + (long long)o * K + k);
    *(half8_t*)(wp + i * 8) = v;
}

}  // namespace

int igemm_patch_num_cfgs() { return kNumPatchCfgs; }

bool igemm_patch_fits(const ConvGeom& g, int cfg) {
    if (cfg < 0 || cfg >= kNumPatchCfgs) return false;
    const PatchCfg& c = kPatchCfgs[cfg];
    // The cooperative patch copy gives each thread one fixed 16-byte piece.
    if ((64 * c.WM * c.WN * c.WK) % (g.C_in / 8) != 0) return false;
    return patch_lds_bytes(g, c) <= 160 * 1024;
}

bool igemm_patch_serves(const ConvGeom& g) {
    const long long xbytes = 2LL * g.N * g.H * g.W * g.C_in, wbytes = 2LL * g.C_out * g.K;
    // C_in <= 448: a patch pixel (C_in*2 + 16 or + 32 bytes) fits one
    // 1 KB load instruction of the loader wave.
    if (g.stride != 1 || g.C_in % 64 != 0 || g.C_in > 448 || xbytes >= (1LL << 31) ||
        wbytes >= (1LL << 31))
        return false;
    for (int i = 0; i < kNumPatchCfgs; ++i)
        if (igemm_patch_fits(g, i)) return true;
    return false;
}

// Busiest CU's tile count times the tile's MFMA work, weighted by LDS bytes
// per MFMA, occupancy, patch stride, ring depth and halo rows; ties go to the
// lower index. The weights were fitted to every tile timed on MI355X over 40
// stride-1 shapes (k 1..5, C_in 64/128, C_out 8..256, 8 x 112 x 112) and the
// 3x3 and 7x7 layers of 28 x 28 and 56 x 56 images: the chosen tile is the
// fastest on 33 of 42 and within 10.2% of it on all, 0.5% slower than the
// fastest tiles summed over the shapes (the earlier, hand-set weights: 10 of
// 42, worst 25%, 7.3% slower summed).
int igemm_patch_choose(const ConvGeom& g) {
    int best = -1;
    double best_cost = 1e300;
    for (int i = 0; i < kNumPatchCfgs; ++i) {
        if (!igemm_patch_fits(g, i)) continue;
        const PatchCfg& c = kPatchCfgs[i];
        const long long tiles = (long long)g.N * ((g.P * g.Q + c.BM - 1) / c.BM) *
                                ((g.C_out + c.BN - 1) / c.BN);
        const long long per_cu = (tiles + 255) / 256;
        // LDS bytes per MFMA of a wave tile: (FM + FN) / (FM * FN).
        const int fm = c.BM / c.WM / 16, fn = c.BN / c.WN / 16;
        const double lds = (double)(fm + fn) / (fm * fn);
        // Two waves per K-group (one per SIMD) expose LDS latency: slower on
        // MI355X despite the lighter LDS traffic. One K-group of four waves
        // has the same single wave per SIMD, which costs when a CU holds one
        // tile; with two or more tiles per CU its smaller workgroups let
        // another tile's waves share the CU, and it is the fastest form.
        double occ = 1.3;
        if (c.WK == 2 && c.WM * c.WN == 4) occ = 1.0;
        else if (c.WK == 1 && c.WM * c.WN == 4) occ = per_cu >= 2 ? 0.85 : 1.15;
        // The dense patch stride costs 2-way bank conflicts on every pixel
        // fragment read (measured: little time); a three-stage ring hides
        // less filter latency.
        const double conflicts = patch_layout(g, c).pstride == g.C_in * 2 + 16 ? 1.05 : 1.0;
        const double ring = c.RING == 3 ? 1.05 : 1.0;
        // Halo: a tile of `rows` output rows copies rows + kh - 1 patch rows.
        const double rows = (double)c.BM / g.Q;
        const double halo = 1.0 + 0.1 * ((rows + g.kh - 1) / rows - 1.0);
        double cost = (double)per_cu * c.BM * c.BN * occ * conflicts * ring * (0.7 + lds) * halo;
        if (cost < best_cost * 0.999) { best = i; best_cost = cost; }
    }
    return best;
}

void igemm_patch_describe(int cfg, int* BM, int* BN, int* WM, int* WN, int* WK, int* ring) {
    const PatchCfg& c = kPatchCfgs[cfg];
    *BM = c.BM; *BN = c.BN; *WM = c.WM; *WN = c.WN; *WK = c.WK; *ring = c.RING;
}

size_t igemm_patch_packed_bytes(const ConvGeom& g, int cfg) {
    if (cfg < 0 || cfg >= kNumPatchCfgs) return 0;
    const size_t nk = (size_t)g.kh * g.kw * (g.C_in / 64), NB = (size_t)(g.C_out + 15) / 16;
    const size_t bytes = nk * NB * 2048;
    return bytes < (1ull << 31) ? bytes : 0;  // 32-bit buffer offsets
}

hipError_t launch_pack_patch_filter(const ConvGeom& g, int cfg, const void* w, void* wp,
                                    hipStream_t s) {
    const size_t bytes = igemm_patch_packed_bytes(g, cfg);
    if (bytes == 0) return hipErrorInvalidValue;
    const long long npieces = (long long)(bytes / 16);
    const int NB = (g.C_out + 15) / 16;
    hipLaunchKernelGGL(pack_patch_filter, dim3((unsigned)((npieces + 255) / 256)), dim3(256), 0,
                       s, (const f16*)w, (f16*)wp, g.C_out, g.K, NB, kPatchCfgs[cfg].WK, npieces);
    return hipGetLastError();
}

hipError_t launch_igemm_patch(const ConvGeom& g, int cfg, int epi, const void* x,
                              const void* w, const float* scale, const float* bias, void* y,
                              hipStream_t s, bool packed) {
    if (!igemm_patch_fits(g, cfg)) return hipErrorInvalidValue;
    if (packed && igemm_patch_packed_bytes(g, cfg) == 0) return hipErrorInvalidValue;
    int i = 0;
#define X(bm, bn, wm, wn, wk, ring)                                                          \
    if (cfg == i)                                                                              \
        return patch_launch_one<bm, bn, wm, wn, wk, ring>(g, epi, x, w, scale, bias, y, packed, \
                                                          s);                                   \
    ++i;
    TG_PATCH_CFGS(X)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace tg
