// train_bn.hip -- BatchNorm with batch statistics (training mode) after the
// convolution, then SiLU.
//
// Batch statistics are a per-channel reduction over every output pixel of
// the batch. "Kernel Fusion" (cheatsheet page) sets this case apart from
// elementwise chains: a reduction with elementwise work fuses into one or two
// passes, but a value that needs results computed by other blocks cannot be
// fused across without a kernel boundary, since there is no grid-wide
// barrier. So the path is:
//   0. the 1x1 layer's kernel (igemm_cu.hip) forms the statistics in its own
//      epilogue from the fp32 accumulators while it writes t1 into y, as
//      (count, mean, sum of squared deviations) per workgroup, and
//      bn_train_finalize_chan combines them (step 3); t1 is then written
//      once and read once. The other kernels take steps 1-4:
//   1. the conv kernel with an identity epilogue writes t1 (y's shape and
//      dtype) into y -- the same kernels as the fused path (api.hip);
//   2. bn_stats_partial: per block of rows, per channel, the sum and the sum
//      of squares of (t1 - shift_c) in fp64, with shift_c = t1[0][c] (one
//      value of the channel: it keeps the sum of squares from cancelling when
//      the mean is large against the spread)
//      (bn_stats_partial_v8 reads 16-byte vectors when the channel count
//      is a multiple of 8);
//   3. bn_train_finalize: per channel, the block partials are added in a
//      fixed order (results do not depend on scheduling); it forms the mean
//      and the biased variance, folds them with gamma, beta and eps into one
//      scale and one bias (as tg_bn_fold does for running statistics), and
//      moves the running estimates by `momentum` (unbiased variance);
//   4. the split form's BatchNorm+SiLU streaming kernel (elementwise.hip)
//      applies scale and bias and SiLU to y in place.
// The batch-normalising transform is the one of Ioffe and Szegedy (2015):
// normalise with the batch mean and the biased batch variance.
#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {
namespace {

constexpr int kStatThreads = 256;  // 4 waves: lane = channel, wave = row phase
constexpr int kStatChans = 64;     // channels per block

// Block (bx, by): rows [bx*R, min(M, bx*R + R)), channels by*64 + lane.
// partial[(bx*C + c)*2 + {0,1}] = sum, sum of squares of (t1 - t1[0][c]).
template <typename T>
__global__ __launch_bounds__(kStatThreads) void bn_stats_partial(const T* __restrict__ t1, int M,
                                                                 int C, int R,
                                                                 double* __restrict__ partial) {
    __shared__ double red[2][kStatThreads / 64][kStatChans];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = blockIdx.y * kStatChans + lane;
    const int r0 = blockIdx.x * R, r1 = r0 + R < M ? r0 + R : M;
    double s1 = 0.0, s2 = 0.0;
    if (c < C) {
        const double shift = (double)to_f32(t1[c]);
        for (int r = r0 + wave; r < r1; r += kStatThreads / 64) {
            const double d = (double)to_f32(t1[(size_t)r * C + c]) - shift;
            s1 += d;
            s2 = __builtin_fma(d, d, s2);
        }
    }
    red[0][wave][lane] = s1;
    red[1][wave][lane] = s2;
    __syncthreads();
    if (wave == 0 && c < C) {
        double a = red[0][0][lane], b = red[1][0][lane];
#pragma unroll
        for (int k = 1; k < kStatThreads / 64; ++k) {
            a += red[0][k][lane];
            b += red[1][k][lane];
        }
        double* p = partial + ((size_t)blockIdx.x * C + c) * 2;
        p[0] = a;
        p[1] = b;
    }
}

// Channel counts that are multiples of 8 (fp16, C <= 4096): a lane reads 16
// bytes (channels 8*cv .. 8*cv+7 of one row); the block's 512 lanes cover RS
// = 512 / CV rows per step (CV = C/8), four steps in flight per lane. The
// lanes' sums are then added per channel in LDS in lane order.
constexpr int kVecThreads = 512;

__global__ __launch_bounds__(kVecThreads) void bn_stats_partial_v8(const half8_t* __restrict__ t1,
                                                                   int M, int C, int R,
                                                                   double* __restrict__ partial) {
    __shared__ double red[kVecThreads][8];
    const int CV = C / 8, RS = kVecThreads / CV;
    const int t = threadIdx.x, cv = t % CV, rp = t / CV;
    const int r0 = blockIdx.x * R, r1 = r0 + R < M ? r0 + R : M;
    double s1[8], s2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s1[e] = s2[e] = 0.0;
    if (rp < RS) {
        const half8_t sh = t1[cv];
        int r = r0 + rp;
        for (; r + 3 * RS < r1; r += 4 * RS) {
            half8_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = t1[(size_t)(r + u * RS) * CV + cv];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double d = (double)(float)v[u][e] - (double)(float)sh[e];
                    s1[e] += d;
                    s2[e] = __builtin_fma(d, d, s2[e]);
                }
        }
        for (; r < r1; r += RS) {
            const half8_t v = t1[(size_t)r * CV + cv];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double d = (double)(float)v[e] - (double)(float)sh[e];
                s1[e] += d;
                s2[e] = __builtin_fma(d, d, s2[e]);
            }
        }
    }
    // Per channel c = 8*cv + e: add the RS lanes (rp = 0 .. RS-1) that hold it.
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[t][e] = pass == 0 ? s1[e] : s2[e];
        __syncthreads();
        for (int c = t; c < C; c += kVecThreads) {
            const int ccv = c / 8, ce = c % 8;
            double a = 0.0;
            for (int k = 0; k < RS; ++k) a += red[k * CV + ccv][ce];
            partial[((size_t)blockIdx.x * C + c) * 2 + pass] = a;
        }
        __syncthreads();
    }
}

// Folds channel c's batch mean and biased variance with gamma, beta and eps
// into one scale and one bias (as tg_bn_fold does for running statistics),
// stores the batch values and moves the running estimates by `momentum`
// (unbiased variance var*M/(M-1)).
__device__ __forceinline__ void bn_train_outputs(int c, int M, double mean, double var,
                                                 const float* gamma, const float* beta, float eps,
                                                 float momentum, float* running_mean,
                                                 float* running_var, float* batch_mean,
                                                 float* batch_var, float* scale, float* bias) {
    const double sc = (double)gamma[c] / sqrt(var + (double)eps);
    scale[c] = (float)sc;
    bias[c] = (float)((double)beta[c] - mean * sc);
    if (batch_mean) batch_mean[c] = (float)mean;
    if (batch_var) batch_var[c] = (float)var;
    if (running_mean) {
        const double m = momentum;
        running_mean[c] = (float)((1.0 - m) * running_mean[c] + m * mean);
        running_var[c] = (float)((1.0 - m) * running_var[c] + m * var * ((double)M / (M - 1)));
    }
}

// One block of 1024 threads per 16 channels: thread t takes channel t % 16
// and adds every 64th row block's partials from block t / 16 on (all its loads
// in flight at once for up to 512 row blocks); the 64 sums of a channel are
// then added in LDS in phase order.
constexpr int kFinChans = 16, kFinPhases = 64;

template <typename T>
__global__ __launch_bounds__(kFinChans * kFinPhases) void bn_train_finalize(
    const T* __restrict__ t1, const double* __restrict__ partial, int GX, int M, int C,
    const float* __restrict__ gamma, const float* __restrict__ beta, float eps, float momentum,
    float* __restrict__ running_mean, float* __restrict__ running_var,
    float* __restrict__ batch_mean, float* __restrict__ batch_var, float* __restrict__ scale,
    float* __restrict__ bias) {
    __shared__ double red[2][kFinPhases][kFinChans];
    const int cl = threadIdx.x % kFinChans, ph = threadIdx.x / kFinChans;
    const int c = blockIdx.x * kFinChans + cl;
    double s1 = 0.0, s2 = 0.0;
    if (c < C) {
        int b = ph;
        for (; b + 7 * kFinPhases < GX; b += 8 * kFinPhases) {
            double a1[8], a2[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                a1[u] = partial[((size_t)(b + u * kFinPhases) * C + c) * 2];
                a2[u] = partial[((size_t)(b + u * kFinPhases) * C + c) * 2 + 1];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                s1 += a1[u];
                s2 += a2[u];
            }
        }
        for (; b < GX; b += kFinPhases) {
            s1 += partial[((size_t)b * C + c) * 2];
            s2 += partial[((size_t)b * C + c) * 2 + 1];
        }
    }
    red[0][ph][cl] = s1;
    red[1][ph][cl] = s2;
    __syncthreads();
    if (ph != 0 || c >= C) return;
    s1 = 0.0;
    s2 = 0.0;
    for (int k = 0; k < kFinPhases; ++k) {
        s1 += red[0][k][cl];
        s2 += red[1][k][cl];
    }
    const double shift = (double)to_f32(t1[c]);
    const double md = s1 / M;                        // mean of (t1 - shift)
    double var = s2 / M - md * md;                   // biased batch variance
    if (var < 0.0) var = 0.0;                        // rounding of an exactly constant channel
    bn_train_outputs(c, M, shift + md, var, gamma, beta, eps, momentum, running_mean, running_var,
                     batch_mean, batch_var, scale, bias);
}

// Triples from the 1x1 and stem kernels' statistics passes: stats[(b*C + c)*3]
// = (count n_b, mean m_b, sum of squared deviations q_b) of workgroup b; four
// channels per workgroup, so the loads spread over C/4 compute units; up to
// kChanHeld * kFinPhases = 1024 workgroups' triples are loaded at once and
// kept in registers for the second pass (the stems' 768: one memory latency
// per channel instead of one per further group of 64). Two
// fixed-order passes (threads (ph, cl) take b = ph, ph + kFinPhases, ...;
// phase 0 then adds the phases in order): the mean from sum(n_b*m_b)/M, then
// the squared deviations as sum(q_b + n_b*(m_b - mean)^2), the exact
// decomposition of the total about the mean. No term cancels and the result
// does not depend on scheduling.
constexpr int kChanChans = 4;   // channels per workgroup of the triple finalize
constexpr int kChanHeld = 16;   // triples a thread keeps in registers between the passes
__global__ __launch_bounds__(kChanChans * kFinPhases) void bn_train_finalize_chan(
    const double* __restrict__ stats, int G, int M, int C, const float* __restrict__ gamma,
    const float* __restrict__ beta, float eps, float momentum, float* __restrict__ running_mean,
    float* __restrict__ running_var, float* __restrict__ batch_mean,
    float* __restrict__ batch_var, float* __restrict__ scale, float* __restrict__ bias) {
    __shared__ double red[kFinPhases][kChanChans];
    __shared__ double mean_s[kChanChans];
    const int cl = threadIdx.x % kChanChans, ph = threadIdx.x / kChanChans;
    const int c = blockIdx.x * kChanChans + cl;
    // Pass 1: sum(n_b*m_b) over this thread's triples b = ph + kFinPhases*i;
    // the first kChanHeld stay in registers for pass 2.
    double hn[kChanHeld], hm[kChanHeld], hq[kChanHeld];
    double a = 0.0;
#pragma unroll
    for (int i = 0; i < kChanHeld; ++i) {
        const int b = ph + i * kFinPhases;
        hn[i] = hm[i] = hq[i] = 0.0;
        if (c < C && b < G) {
            const double* t = stats + ((size_t)b * C + c) * 3;
            hn[i] = t[0];
            hm[i] = t[1];
            hq[i] = t[2];
        }
    }
#pragma unroll
    for (int i = 0; i < kChanHeld; ++i) a += hn[i] * hm[i];
    if (c < C)
        for (int b = ph + kChanHeld * kFinPhases; b < G; b += kFinPhases) {
            const double* t = stats + ((size_t)b * C + c) * 3;
            a += t[0] * t[1];
        }
    red[ph][cl] = a;
    __syncthreads();
    if (ph == 0) {
        double s = 0.0;
        for (int k = 0; k < kFinPhases; ++k) s += red[k][cl];
        mean_s[cl] = s / M;
    }
    __syncthreads();
    const double mean = mean_s[cl];
    // Pass 2: sum(q_b + n_b*(m_b - mean)^2).
    a = 0.0;
#pragma unroll
    for (int i = 0; i < kChanHeld; ++i) {
        const double d = hm[i] - mean;
        a += hq[i] + hn[i] * d * d;
    }
    if (c < C)
        for (int b = ph + kChanHeld * kFinPhases; b < G; b += kFinPhases) {
            const double* t = stats + ((size_t)b * C + c) * 3;
            const double d = t[1] - mean;
            a += t[2] + t[0] * d * d;
        }
    __syncthreads();
    red[ph][cl] = a;
    __syncthreads();
    if (ph != 0 || c >= C) return;
    double q = 0.0;
    for (int k = 0; k < kFinPhases; ++k) q += red[k][cl];
    bn_train_outputs(c, M, mean, q / M, gamma, beta, eps, momentum, running_mean, running_var,
                     batch_mean, batch_var, scale, bias);
}

}  // namespace

size_t bn_train_chan_bytes(int G, int C) { return (size_t)G * C * 3 * sizeof(double); }

hipError_t launch_bn_train_finalize_chan(const double* stats, int G, int M, int C,
                                         const float* gamma, const float* beta, float eps,
                                         float momentum, float* running_mean, float* running_var,
                                         float* batch_mean, float* batch_var, float* scale,
                                         float* bias, hipStream_t s) {
    hipLaunchKernelGGL(bn_train_finalize_chan, dim3((C + kChanChans - 1) / kChanChans),
                       dim3(kChanChans * kFinPhases), 0, s, stats, G, M, C, gamma, beta, eps,
                       momentum, running_mean, running_var, batch_mean, batch_var, scale, bias);
    return hipGetLastError();
}

void bn_train_grid(int M, int* R, int* GX) {
    // About 512 row blocks (two per compute unit), at least 64 rows each.
    int r = (M + 511) / 512;
    if (r < 64) r = 64;
    *R = r;
    *GX = (M + r - 1) / r;
}

size_t bn_train_partial_bytes(int M, int C) {
    int R, GX;
    bn_train_grid(M, &R, &GX);
    return (size_t)GX * C * 2 * sizeof(double);
}

hipError_t launch_bn_train_stats(bool f32, const void* t1, int M, int C, const float* gamma,
                                 const float* beta, float eps, float momentum,
                                 float* running_mean, float* running_var, float* batch_mean,
                                 float* batch_var, double* partial, float* scale, float* bias,
                                 hipStream_t s) {
    int R, GX;
    bn_train_grid(M, &R, &GX);
    const dim3 grid(GX, (C + kStatChans - 1) / kStatChans), fin((C + kFinChans - 1) / kFinChans);
    const bool v8 = !f32 && C % 8 == 0 && C <= 8 * kVecThreads && ((uintptr_t)t1 & 15) == 0;
    if (v8) {
        hipLaunchKernelGGL(bn_stats_partial_v8, dim3(GX), dim3(kVecThreads), 0, s,
                           (const half8_t*)t1, M, C, R, partial);
        hipLaunchKernelGGL(bn_train_finalize<f16>, fin, dim3(kFinChans * kFinPhases), 0, s, (const f16*)t1,
                           (const double*)partial, GX, M, C, gamma, beta, eps, momentum,
                           running_mean, running_var, batch_mean, batch_var, scale, bias);
    } else if (f32) {
        hipLaunchKernelGGL(bn_stats_partial<float>, grid, dim3(kStatThreads), 0, s,
                           (const float*)t1, M, C, R, partial);
        hipLaunchKernelGGL(bn_train_finalize<float>, fin, dim3(kFinChans * kFinPhases), 0, s, (const float*)t1,
                           (const double*)partial, GX, M, C, gamma, beta, eps, momentum,
                           running_mean, running_var, batch_mean, batch_var, scale, bias);
    } else {
        hipLaunchKernelGGL(bn_stats_partial<f16>, grid, dim3(kStatThreads), 0, s, (const f16*)t1,
                           M, C, R, partial);
        hipLaunchKernelGGL(bn_train_finalize<f16>, fin, dim3(kFinChans * kFinPhases), 0, s, (const f16*)t1,
                           (const double*)partial, GX, M, C, gamma, beta, eps, momentum,
                           running_mean, running_var, batch_mean, batch_var, scale, bias);
    }
    return hipGetLastError();
}

}  // namespace tg
