// layout.hip -- layout conversions around the channels-last path.
//
// "When the fusion you want is impossible, fuse into the producer" (layout
// paragraph): storing the filters channels-last once, at load time, deleted
// the per-call NCHW<->NHWC conversion kernels of a convolution pipeline with
// bit-identical output. This library's kernels take x and y NHWC and w OHWI;
// a caller holding PyTorch-layout tensors (NCHW activations, OIHW filters)
// converts the filters once with tg_filter_oihw_to_ohwi and, if its
// activations stay NCHW, pays two conversion legs per call
// (tg_nchw_to_nhwc on x, tg_nhwc_to_nchw on y), which the benchmark measures.
//
// All three are one batched transpose, dst[b][j][i] = src[b][i][j]: in
// 64 x 64 tiles through LDS so that both the reads and the writes run along
// contiguous rows, or, when one side has at most 16 entries (3-channel
// images, filter taps), one thread per row or column; a pure permutation, so
// bit-exact for any dtype.
#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {
namespace {

constexpr int kTile = 64;

// src [B][R][S] -> dst [B][S][R]. Block = 256 threads (64 x 4) per tile;
// blockIdx.x enumerates (b, tile row, tile column).
template <typename T>
__global__ __launch_bounds__(256) void transpose_tiles(const T* __restrict__ src,
                                                       T* __restrict__ dst, int R, int S,
                                                       int tiles_r, int tiles_s) {
    __shared__ T tile[kTile][kTile + 1];
    const int per_b = tiles_r * tiles_s;
    const int b = blockIdx.x / per_b, rem = blockIdx.x - b * per_b;
    const int tr = rem / tiles_s, ts = rem - tr * tiles_s;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const size_t base = (size_t)b * R * S;
    const int r0 = tr * kTile, s0 = ts * kTile;
    // read rows r0 + i of src along s (contiguous)
#pragma unroll 4
    for (int i = ty; i < kTile; i += 4) {
        const int r = r0 + i, s = s0 + tx;
        if (r < R && s < S) tile[i][tx] = src[base + (size_t)r * S + s];
    }
    __syncthreads();
    // write rows s0 + i of dst along r (contiguous)
#pragma unroll 4
    for (int i = ty; i < kTile; i += 4) {
        const int s = s0 + i, r = r0 + tx;
        if (s < S && r < R) dst[base + (size_t)s * R + r] = tile[tx][i];
    }
}

// Few rows (R <= 16, e.g. the 3 channels of an RGB image going NCHW ->
// NHWC): one thread per (b, s) gathers the R values of its column -- each
// read instruction runs along s across the wave -- and writes them as one
// contiguous group.
template <typename T>
__global__ __launch_bounds__(256) void transpose_few_rows(const T* __restrict__ src,
                                                          T* __restrict__ dst, int B, int R,
                                                          int S) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long long)B * S) return;
    const long long b = i / S, sidx = i - b * S;
    const T* sp = src + b * R * S + sidx;
    T* dp = dst + i * R;
    for (int r = 0; r < R; ++r) dp[r] = sp[(long long)r * S];
}

// Few columns (S <= 16, e.g. NHWC -> NCHW of a 3-channel tensor, or the
// kh*kw taps of a filter): one thread per (b, r) reads its contiguous row
// and scatters it, each write instruction running along r across the wave.
template <typename T>
__global__ __launch_bounds__(256) void transpose_few_cols(const T* __restrict__ src,
                                                          T* __restrict__ dst, int B, int R,
                                                          int S) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long long)B * R) return;
    const long long b = i / R, r = i - b * R;
    const T* sp = src + i * S;
    T* dp = dst + b * R * S + r;
    for (int c = 0; c < S; ++c) dp[(long long)c * R] = sp[c];
}

template <typename T>
hipError_t transpose_t(const T* src, T* dst, int B, int R, int S, hipStream_t s) {
    if (R <= 16 || S <= 16) {
        const long long n = (long long)B * (R <= 16 ? S : R);
        const long long blocks = (n + 255) / 256;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        if (R <= 16)
            hipLaunchKernelGGL(transpose_few_rows<T>, dim3((unsigned)blocks), dim3(256), 0, s, src,
                               dst, B, R, S);
        else
            hipLaunchKernelGGL(transpose_few_cols<T>, dim3((unsigned)blocks), dim3(256), 0, s, src,
                               dst, B, R, S);
        return hipGetLastError();
    }
    const int tiles_r = (R + kTile - 1) / kTile, tiles_s = (S + kTile - 1) / kTile;
    const long long blocks = (long long)B * tiles_r * tiles_s;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(transpose_tiles<T>, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, R, S,
                       tiles_r, tiles_s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_transpose(bool f32, const void* src, void* dst, int B, int R, int S,
                            hipStream_t s) {
    if (f32) return transpose_t((const float*)src, (float*)dst, B, R, S, s);
    return transpose_t((const f16*)src, (f16*)dst, B, R, S, s);
}

}  // namespace tg
