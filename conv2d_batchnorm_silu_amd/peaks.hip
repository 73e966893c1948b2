// peaks.hip -- microbenchmarks of the MI355X rates the fused kernels are
// measured against: HBM streaming (copy, read-only, write-only with and
// without the non-temporal hint), fp16 MFMA throughput (16x16x32 and
// 32x32x16 forms, one or two waves per SIMD) and LDS read bandwidth
// (ds_read_b128, conflict-free). Built into its own library (libtgpeaks.so)
// by peaks.py, which launches these kernels and times them with HIP events;
// nothing in the fused-kernel library depends on it.
//
// The roofline of each workload is the published peak (HBM 8 TB/s, dense
// fp16 MFMA 2.5 PFLOP/s); these measured rates show how much of it a
// streaming or matrix kernel can reach on this part ("Costs and benefits of
// kernel fusion": the traffic a fusion removes is worth what the memory
// system actually delivers, not its peak).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 pk_half8 __attribute__((ext_vector_type(8)));
typedef float pk_float4 __attribute__((ext_vector_type(4)));
typedef float pk_float16 __attribute__((ext_vector_type(16)));
typedef uint32_t pk_u32x4 __attribute__((ext_vector_type(4)));

// ---- HBM ----------------------------------------------------------------
// Grid-stride loops over 16-byte elements.
__global__ void pk_copy(const pk_u32x4* __restrict__ src, pk_u32x4* __restrict__ dst, long long n) {
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

__global__ void pk_read(const pk_u32x4* __restrict__ src, long long n, unsigned* out) {
    pk_u32x4 s = {0, 0, 0, 0};
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        s ^= src[i];
    if ((s[0] ^ s[1] ^ s[2] ^ s[3]) == 0x9e3779b9u) out[0] = 1;  // keeps the loads
}

template <bool NT>
__global__ void pk_write(pk_u32x4* __restrict__ dst, long long n) {
    const pk_u32x4 v = {(unsigned)threadIdx.x, 1u, 2u, 3u};
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x) {
        if constexpr (NT) __builtin_nontemporal_store(v, dst + i);
        else dst[i] = v;
    }
}

// Copy whose reads are direct-to-LDS buffer loads (the fused kernels' way of
// reading x): each wave moves 1 KB per step, global -> LDS (lane l's 16
// bytes land at the wave's slot + 16*l), then each lane stores the slot it
// loaded. The lane reads only what its own load wrote, so the wave's own
// vector-memory count orders the two. A calibration kernel for the HBM
// byte counters of such reads.
__global__ __launch_bounds__(256) void pk_copy_dma(const pk_u32x4* __restrict__ src,
                                                   pk_u32x4* __restrict__ dst, long long n) {
    __shared__ pk_u32x4 slot[256];
    const unsigned long long a = (unsigned long long)src;
    pk_u32x4 rs;
    rs[0] = (unsigned)a;
    rs[1] = (unsigned)(a >> 32) & 0xffffu;
    rs[2] = (unsigned)(n * 16);
    rs[3] = 0x00020000u;
    const int wave = threadIdx.x >> 6;
    const unsigned lds = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)((__attribute__((address_space(3))) pk_u32x4*)slot) + wave * 1024u);
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x) {
        const unsigned voff = (unsigned)(i * 16);
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds\n\ts_waitcnt vmcnt(0)"
                     :
                     : "v"(voff), "s"(rs), "{m0}"(lds)
                     : "memory");
        dst[i] = slot[threadIdx.x];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}

// Latency of a batch of N 1 KB loads from one wave (64 lanes x 16 bytes):
// direct-to-LDS (MODE 0, every load of a wave into its own 1 KB slot) or
// into registers (MODE 1), then a wait for all of them, `iters` times. The
// source window is `window` bytes (a small window stays in L2; a large one
// streams from HBM), each load a new 1 KB of it. Time per batch against N
// tells whether one wave's loads overlap or follow one another.
template <int MODE, int N>
__global__ __launch_bounds__(512) void pk_vmem_batch(const unsigned char* __restrict__ src,
                                                     unsigned long long window, int iters,
                                                     float* out) {
    __shared__ __attribute__((aligned(16))) unsigned char slot[8 * 1024];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long long a = (unsigned long long)src;
    pk_u32x4 rs;
    rs[0] = (unsigned)a;
    rs[1] = (unsigned)(a >> 32) & 0xffffu;
    rs[2] = 0xffffffffu;
    rs[3] = 0x00020000u;
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, -1, 0x00020000);
    const unsigned lds = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)slot) + wave * 1024u);
    const unsigned long long kb = window / 1024;
    unsigned long long k = ((unsigned long long)blockIdx.x * (blockDim.x >> 6) + wave) * 7919ull;
    pk_u32x4 acc = {0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
        if (MODE == 0) {
#pragma unroll
            for (int j = 0; j < N; ++j) {
                const unsigned voff = (unsigned)(((k + j) % kb) * 1024 + lane * 16);
                asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                             :
                             : "v"(voff), "s"(rs), "{m0}"(lds)
                             : "memory");
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else {
            pk_u32x4 v[N];
#pragma unroll
            for (int j = 0; j < N; ++j) {
                const unsigned voff = (unsigned)(((k + j) % kb) * 1024 + lane * 16);
                v[j] = __builtin_bit_cast(pk_u32x4,
                                          __builtin_amdgcn_raw_buffer_load_b128(rb, voff, 0, 0));
            }
#pragma unroll
            for (int j = 0; j < N; ++j) acc ^= v[j];
        }
        k += N;
    }
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) out[0] = 1.f;
}

// ---- MFMA ---------------------------------------------------------------
// Each wave runs `iters` rounds of ACC independent MFMAs (no dependency
// between consecutive instructions), so the matrix core is the only limit.
template <int ACC>
__global__ __launch_bounds__(512) void pk_mfma16(int iters, float* out) {
    pk_half8 a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = (_Float16)(0.001f * (threadIdx.x + e));
        b[e] = (_Float16)(0.002f * (threadIdx.x - e));
    }
    pk_float4 acc[ACC];
    for (int u = 0; u < ACC; ++u) acc[u] = (pk_float4){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int u = 0; u < ACC; ++u)
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[u], 0, 0, 0);
    float s = 0.f;
    for (int u = 0; u < ACC; ++u) s += acc[u][0] + acc[u][1] + acc[u][2] + acc[u][3];
    if (s == 12345.678f) out[0] = s;
}

template <int ACC>
__global__ __launch_bounds__(512) void pk_mfma32(int iters, float* out) {
    pk_half8 a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = (_Float16)(0.001f * (threadIdx.x + e));
        b[e] = (_Float16)(0.002f * (threadIdx.x - e));
    }
    pk_float16 acc[ACC];
    for (int u = 0; u < ACC; ++u)
        for (int e = 0; e < 16; ++e) acc[u][e] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int u = 0; u < ACC; ++u)
            acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[u], 0, 0, 0);
    float s = 0.f;
    for (int u = 0; u < ACC; ++u)
        for (int e = 0; e < 16; ++e) s += acc[u][e];
    if (s == 12345.678f) out[0] = s;
}

// ---- LDS ----------------------------------------------------------------
// Every lane reads 16 bytes per ds_read_b128 from 16-byte slot l of a 1 KB
// row (a conflict-free pattern), 8 reads in flight per wait; the reads are
// inline assembly so that none of them is folded away.
__global__ __launch_bounds__(512) void pk_lds(int iters, float* out) {
    __shared__ pk_half8 buf[2048];  // 32 KB
    for (int i = threadIdx.x; i < 2048; i += blockDim.x)
        for (int e = 0; e < 8; ++e) buf[i][e] = (_Float16)(i + e);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned base = (unsigned)(uintptr_t)(
        (__attribute__((address_space(3))) pk_half8*)buf) + (unsigned)lane * 16u;
    pk_half8 s = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
        pk_half8 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const unsigned addr = base + (unsigned)(((it * 8 + u + wave * 4) & 31) * 1024);
            asm volatile("ds_read_b128 %0, %1" : "=v"(v[u]) : "v"(addr));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    if ((float)s[0] == 12345.678f) out[0] = (float)s[1];
}

// Fragment-read pattern of the implicit-GEMM kernels: lane l reads 16 bytes
// at (l % 16) * stride + (l / 16) * 16 -- sixteen rows (pixels or filter
// rows) of `stride` bytes, four 16-byte pieces each -- 8 reads of distinct
// row blocks in flight per wait. Measures how the row stride maps onto the
// LDS banks.
__global__ __launch_bounds__(512) void pk_lds_stride(int iters, int stride, float* out) {
    extern __shared__ __attribute__((aligned(16))) unsigned char pk_dyn[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 16 * stride * 8 / 16; i += blockDim.x)
        ((pk_u32x4*)pk_dyn)[i] = (pk_u32x4){(unsigned)i, 0u, 0u, 0u};
    __syncthreads();
    const unsigned base = (unsigned)(uintptr_t)(
        (__attribute__((address_space(3))) unsigned char*)pk_dyn) +
        (unsigned)((lane & 15) * stride + (lane >> 4) * 16);
    pk_half8 s = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
        pk_half8 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const unsigned addr = base + (unsigned)((((it + u + wave) & 7)) * 16 * stride);
            asm volatile("ds_read_b128 %0, %1" : "=v"(v[u]) : "v"(addr));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    if ((float)s[0] == 12345.678f) out[0] = (float)s[1];
}

// LDS read patterns of the implicit-GEMM fragments. Each of 8 waves issues
// 12 ds_read_b128 back to back per iteration, 4 KB apart (the same bank
// alignment), then waits; lane l = 16 p + r (row r, piece p) reads at byte
// offset:
//   0  16 l                                   (linear: every bank once per 16 lanes)
//   1  r * prm + 16 p                         (16 pixels of a patch, pixel stride prm)
//   2  (r + (r >= 8 ? 6 : 0)) * prm + 16 p    (... wrapping to the next row after 8)
//   3  64 r + 16 (p ^ ((r >> 1) & 3))         (64-byte filter rows, three swizzles)
//   4  64 r + 16 (p ^ ((r >> 2) & 3))
//   5  64 r + 16 (p ^ (((r >> 1) ^ (r >> 2)) & 3))
//   6  128 r + 16 ((p + 4 prm) ^ ((r >> 1) & 7))      (128-byte filter rows,
//   7  128 r + 16 ((p + 4 prm) ^ ((r & 7) ^ (r >> 3)))  half prm of the row)
// Bytes per clock per CU against the linear pattern show the bank conflicts
// of each layout.
constexpr int kPatReads = 12, kPatStep = 4096, kPatLds = 96 * 1024;
__global__ __launch_bounds__(512) void pk_lds_pattern(int iters, int mode, int prm, float* out) {
    extern __shared__ __attribute__((aligned(16))) unsigned char pk_dyn[];
    for (int i = threadIdx.x; i < kPatLds / 16; i += blockDim.x)
        ((pk_u32x4*)pk_dyn)[i] = (pk_u32x4){(unsigned)i, 3u, 5u, 7u};
    __syncthreads();
    const int lane = threadIdx.x & 63, r = lane & 15, p = lane >> 4;
    int off;
    switch (mode) {
        case 0: off = 16 * lane; break;
        case 1: off = r * prm + 16 * p; break;
        case 2: off = (r + (r >= 8 ? 6 : 0)) * prm + 16 * p; break;
        case 3: off = 64 * r + 16 * (p ^ ((r >> 1) & 3)); break;
        case 4: off = 64 * r + 16 * (p ^ ((r >> 2) & 3)); break;
        case 5: off = 64 * r + 16 * (p ^ (((r >> 1) ^ (r >> 2)) & 3)); break;
        case 6: off = 128 * r + 16 * ((p + 4 * prm) ^ ((r >> 1) & 7)); break;
        default: off = 128 * r + 16 * ((p + 4 * prm) ^ ((r & 7) ^ (r >> 3))); break;
    }
    const unsigned base = (unsigned)(uintptr_t)(
        (__attribute__((address_space(3))) unsigned char*)pk_dyn) + (unsigned)off;
    unsigned addr[kPatReads];
#pragma unroll
    for (int u = 0; u < kPatReads; ++u) addr[u] = base + (unsigned)(u * kPatStep);
    pk_u32x4 acc = {0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
        pk_u32x4 v[kPatReads];
#pragma unroll
        for (int u = 0; u < kPatReads; ++u)
            asm volatile("ds_read_b128 %0, %1" : "=v"(v[u]) : "v"(addr[u]));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int u = 0; u < kPatReads; ++u) acc ^= v[u];
    }
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) out[0] = 1.f;
}

// The implicit-GEMM step shape: per wave a 4 x 7 grid of 16x16x32 MFMAs
// (4 filter fragments held in registers, 7 pixel fragments) with the next
// step's 7 pixel fragments read from LDS (16 rows of a 160-byte stride,
// four 16-byte pieces each) during the first 7 MFMAs and waited for at the
// end of the step. MODE 0 leaves the reads out; MODE 2 also reloads each
// filter fragment from global memory (a 4 KB, cache-resident table, one
// contiguous kilobyte per load) right after its last MFMA of the step, for
// use two steps later. Reports the time per step against the MFMAs alone.
template <int MODE>
__global__ __launch_bounds__(256) void pk_mfma_lds(int iters, const pk_half8* __restrict__ g,
                                                   float* out) {
    __shared__ __attribute__((aligned(16))) unsigned char buf[7 * 16 * 160 * 2];
    for (int i = threadIdx.x; i < (int)sizeof(buf) / 16; i += blockDim.x)
        ((pk_u32x4*)buf)[i] = (pk_u32x4){(unsigned)i, 1u, 2u, 3u};
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const unsigned base = (unsigned)(uintptr_t)(
        (__attribute__((address_space(3))) unsigned char*)buf) +
        (unsigned)((lane & 15) * 160 + (lane >> 4) * 16);
    pk_half8 a[4], a1[4], b0[7], b1[7];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i][e] = (_Float16)(0.001f * (threadIdx.x + e + i));
            a1[i][e] = (_Float16)(0.004f * (threadIdx.x + e + i));
        }
#pragma unroll
        for (int j = 0; j < 7; ++j) {
            b0[j][e] = (_Float16)(0.002f * (threadIdx.x - e + j));
            b1[j][e] = (_Float16)(0.003f * (threadIdx.x - e + j));
        }
    }
    pk_float4 acc[4][7];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 7; ++j) acc[i][j] = (pk_float4){0.f, 0.f, 0.f, 0.f};
    auto step = [&](pk_half8 (&ai)[4], pk_half8 (&bc)[7], pk_half8 (&bn)[7], unsigned half) {
#pragma unroll
        for (int f = 0; f < 28; ++f) {
            const int i = f / 7, j = f % 7;
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ai[i], bc[j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (MODE >= 1 && f < 7)
                asm volatile("ds_read_b128 %0, %1" : "=v"(bn[f]) : "v"(base + half + f * 2560u));
            if (MODE == 2 && j == 6) ai[i] = g[i * 64 + lane + (half ? 0 : 256)];
            __builtin_amdgcn_sched_barrier(0);
        }
        if (MODE >= 1) {
#pragma unroll
            for (int j = 0; j < 7; ++j) asm volatile("" : "+v"(bn[j]));
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
    };
    for (int it = 0; it < iters; ++it) {
        step(a, b0, b1, 0u);
        if constexpr (MODE == 2) step(a1, b1, b0, 7u * 2560u);
        else step(a, b1, b0, 7u * 2560u);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 7; ++j) s += acc[i][j][0] + acc[i][j][3];
    if (s == 12345.678f) out[0] = s;
}

// ---- VALU and transcendental unit ------------------------------------------
// Eight independent chains per lane of one operation: 0 = v_fma_f32,
// 1 = v_exp_f32, 2 = v_rcp_f32; the result feeds the next step of its chain.
// Rates are lane-operations per second; the epilogue's activation costs one
// exp and one reciprocal per output.
template <int OP>
__global__ __launch_bounds__(512) void pk_valu(int iters, float* out) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = 0.5f + 0.001f * (float)(threadIdx.x + u);
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if constexpr (OP == 0) v[u] = __builtin_fmaf(v[u], 0.999f, 0.0001f);
            else if constexpr (OP == 1) v[u] = __builtin_amdgcn_exp2f(v[u]) * -0.25f;
            else v[u] = __builtin_amdgcn_rcpf(v[u]) + 0.5f;
        }
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
    if (s == 12345.678f) out[0] = s;
}

extern "C" {

// mode 0: MFMAs only; 1: with the pixel-fragment LDS reads; 2: also the
// filter-fragment global loads. Two steps
// (56 MFMAs per wave) per iteration; 256 threads per block.
// g: 8 KB of device memory (mode 2 reads it).
int tgp_mfma_lds(int mode, int iters, int grid, const void* g, void* out, void* stream) {
    const pk_half8* gp = (const pk_half8*)g;
    if (mode == 0)
        hipLaunchKernelGGL(pk_mfma_lds<0>, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters,
                           gp, (float*)out);
    else if (mode == 1)
        hipLaunchKernelGGL(pk_mfma_lds<1>, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters,
                           gp, (float*)out);
    else
        hipLaunchKernelGGL(pk_mfma_lds<2>, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters,
                           gp, (float*)out);
    return (int)hipGetLastError();
}

// op: 0 fma, 1 exp, 2 rcp (8 operations per lane and iteration).
int tgp_valu(int op, int iters, int grid, int block, void* out, void* stream) {
    if (op == 0)
        hipLaunchKernelGGL(pk_valu<0>, dim3(grid), dim3(block), 0, (hipStream_t)stream, iters,
                           (float*)out);
    else if (op == 1)
        hipLaunchKernelGGL(pk_valu<1>, dim3(grid), dim3(block), 0, (hipStream_t)stream, iters,
                           (float*)out);
    else
        hipLaunchKernelGGL(pk_valu<2>, dim3(grid), dim3(block), 0, (hipStream_t)stream, iters,
                           (float*)out);
    return (int)hipGetLastError();
}

// Launchers: each returns the hipError_t of the launch. Grids and blocks are
// the caller's (peaks.py documents what it uses).
int tgp_copy(const void* src, void* dst, long long bytes, int grid, void* stream) {
    hipLaunchKernelGGL(pk_copy, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const pk_u32x4*)src, (pk_u32x4*)dst, bytes / 16);
    return (int)hipGetLastError();
}

// bytes: a multiple of 16 below 4 GiB; grid x 256 lanes move 16 bytes each per step.
int tgp_copy_dma(const void* src, void* dst, long long bytes, int grid, void* stream) {
    if (bytes % 16 != 0 || bytes >= (1LL << 32)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(pk_copy_dma, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const pk_u32x4*)src, (pk_u32x4*)dst, bytes / 16);
    return (int)hipGetLastError();
}

int tgp_read(const void* src, long long bytes, void* out, int grid, void* stream) {
    hipLaunchKernelGGL(pk_read, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const pk_u32x4*)src, bytes / 16, (unsigned*)out);
    return (int)hipGetLastError();
}

int tgp_write(void* dst, long long bytes, int nt, int grid, void* stream) {
    if (nt)
        hipLaunchKernelGGL(pk_write<true>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                           (pk_u32x4*)dst, bytes / 16);
    else
        hipLaunchKernelGGL(pk_write<false>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                           (pk_u32x4*)dst, bytes / 16);
    return (int)hipGetLastError();
}

// shape 0: 16x16x32 (16384 FLOP per instruction), 1: 32x32x16 (32768).
// block = 64 * waves per workgroup; 8 (16x16x32) or 4 (32x32x16)
// independent accumulators per wave.
int tgp_mfma(int shape, int iters, int grid, int block, void* out, void* stream) {
    if (shape == 0)
        hipLaunchKernelGGL(pk_mfma16<8>, dim3(grid), dim3(block), 0, (hipStream_t)stream, iters,
                           (float*)out);
    else
        hipLaunchKernelGGL(pk_mfma32<4>, dim3(grid), dim3(block), 0, (hipStream_t)stream, iters,
                           (float*)out);
    return (int)hipGetLastError();
}

// stride: bytes between the 16 rows of one read (16 * 8 * stride bytes of
// dynamic LDS, at most 160 KB).
int tgp_lds_stride(int iters, int stride, int grid, int block, void* out, void* stream) {
    const size_t lds = (size_t)16 * 8 * stride;
    if (stride < 64 || stride % 16 != 0 || lds > 160 * 1024) return (int)hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute((const void*)pk_lds_stride,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(pk_lds_stride, dim3(grid), dim3(block), lds, (hipStream_t)stream, iters,
                       stride, (float*)out);
    return (int)hipGetLastError();
}

// One workgroup of 512 threads per CU (96 KB of LDS each); mode and prm as
// in pk_lds_pattern: prm 16..512 in steps of 16 for modes 1-2, 0 or 1 for
// modes 6-7 (every address stays inside the 96 KB).
int tgp_lds_pattern(int iters, int mode, int prm, int grid, void* out, void* stream) {
    if (mode < 0 || mode > 7) return (int)hipErrorInvalidValue;
    if ((mode == 1 || mode == 2) && (prm < 16 || prm > 512 || prm % 16 != 0))
        return (int)hipErrorInvalidValue;
    if (mode >= 6 && prm != 0 && prm != 1) return (int)hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute((const void*)pk_lds_pattern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kPatLds);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(pk_lds_pattern, dim3(grid), dim3(512), kPatLds, (hipStream_t)stream, iters,
                       mode, prm, (float*)out);
    return (int)hipGetLastError();
}

// mode 0: direct-to-LDS, 1: into registers; n = 1, 4 or 16 loads per
// batch; waves per workgroup 1..8; window: bytes of src, a multiple of 1 KB
// and below 4 GB (every offset stays inside it).
int tgp_vmem_batch(int mode, int n, const void* src, unsigned long long window, int iters,
                   int grid, int waves, void* out, void* stream) {
    if (waves < 1 || waves > 8 || window < 1024 || window % 1024 || window >= (1ull << 32))
        return (int)hipErrorInvalidValue;
    const dim3 g(grid), b(64 * waves);
    hipStream_t s = (hipStream_t)stream;
    const unsigned char* p = (const unsigned char*)src;
#define TG_VB(M, NN)                                                                        \
    if (mode == M && n == NN) {                                                             \
        hipLaunchKernelGGL((pk_vmem_batch<M, NN>), g, b, 0, s, p, window, iters, (float*)out); \
        return (int)hipGetLastError();                                                      \
    }
    TG_VB(0, 1) TG_VB(0, 4) TG_VB(0, 16) TG_VB(1, 1) TG_VB(1, 4) TG_VB(1, 16)
#undef TG_VB
    return (int)hipErrorInvalidValue;
}

int tgp_lds(int iters, int grid, int block, void* out, void* stream) {
    hipLaunchKernelGGL(pk_lds, dim3(grid), dim3(block), 0, (hipStream_t)stream, iters,
                       (float*)out);
    return (int)hipGetLastError();
}

}  // extern "C"
