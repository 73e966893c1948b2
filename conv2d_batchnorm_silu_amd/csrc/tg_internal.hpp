// tg_internal.hpp -- host-side types shared by the plan/ABI code and the
// kernel launchers. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace tg {

// Convolution geometry. Every element count of x, w and y is below 2^31
// (checked at plan creation), so int offsets suffice inside the kernels.
struct ConvGeom {
    int N, H, W, C_in, C_out, kh, kw, stride, pad;
    int P, Q;  // output extent
    int M;     // N * P * Q output pixels
    int K;     // kh * kw * C_in reduction length
    int out8;  // 1: y is fp8 (E4M3), one byte per element; 0: y in the input dtype
    // Residual added to the epilogue's output (y's shape and dtype), or null.
    // Set per call (tg_conv_bn_silu_run_residual), never in a plan.
    const void* res;
};

// Implicit-GEMM tile variants compiled into the library (see igemm.hip).
// BM pixels x BN channels per workgroup of 256 threads (4 wavefronts arranged
// WM x WN); the reduction is staged through LDS BK halves at a time.
struct IgemmCfg {
    int BM, BN, BK, WM, WN;
    int WK = 1;  // K-groups of 4 waves splitting each chunk (direct-to-LDS variant)
};
int igemm_num_cfgs();
const IgemmCfg& igemm_cfg(int i);

// Tiled direct kernel parameters chosen at plan time.
struct TiledCfg {
    int R;          // output rows per workgroup
    int WPad;       // staged input columns per row, (Q-1)*stride + kw
    int lds_bytes;  // dynamic LDS per workgroup
};
// Largest band that fits; returns false when the shape cannot be served.
bool tiled_plan(const ConvGeom& g, TiledCfg* out);

// Raise `kernel`'s dynamic-LDS limit on the current device to at least
// `bytes` (hipFuncSetAttribute), once per kernel, device and size. Safe when
// several host threads launch concurrently: the record of limits already set
// is guarded by a mutex.
hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes);

hipError_t launch_scalar(const ConvGeom& g, bool f32, int epi, const void* x, const void* w,
                         const float* scale, const float* bias, void* y, hipStream_t s);
hipError_t launch_tiled(const ConvGeom& g, const TiledCfg& c, int epi, const void* x,
                        const void* w, const float* scale, const float* bias, void* y,
                        hipStream_t s);
hipError_t launch_igemm(const ConvGeom& g, int cfg, int epi, const void* x, const void* w,
                        const float* scale, const float* bias, void* y, hipStream_t s);
// Register-resident-weights implicit GEMM (igemm_rw.hip): K <= 64, C_out <= 256.
bool igemm_rw_serves(const ConvGeom& g);
void igemm_rw_choose(const ConvGeom& g, int* nf, int* cs, int* ncw);
bool igemm_rw_valid(const ConvGeom& g, int nf, int cs, int ncw);
int igemm_rw_grid(const ConvGeom& g, int slots);
hipError_t launch_igemm_rw(const ConvGeom& g, int grid, int nf, int cs, int ncw, bool nt,
                           int epi, const void* x, const void* w, const float* scale,
                           const float* bias, void* y, hipStream_t s);
hipError_t launch_igemm_stream(const ConvGeom& g, int waves_per_cu, int xdma, bool nt, int epi,
                               const void* x, const void* w, const float* scale,
                               const float* bias, void* y, hipStream_t s);

// One persistent workgroup per compute unit (igemm_cu.hip): 1x1, stride 1,
// unpadded, C_in == 64, C_out a multiple of 64 up to 256. nwaves is a
// multiple of C_out/64 (at most 16); pd is the input prefetch depth (1..3).
bool igemm_cu_serves(const ConvGeom& g);
int igemm_cu_waves(const ConvGeom& g, int per_group);
hipError_t launch_igemm_cu(const ConvGeom& g, int nwaves, int pd, bool nt, int epi,
                           const void* x, const void* w, const float* scale, const float* bias,
                           void* y, hipStream_t s);
// Direct-to-LDS pipelined implicit GEMM (igemm_dma.hip): C_in % 64 == 0.
bool igemm_dma_serves(const ConvGeom& g);
int igemm_dma_num_cfgs();
const IgemmCfg& igemm_dma_cfg(int i);
hipError_t launch_igemm_dma(const ConvGeom& g, int cfg, int epi, const void* x,
                            const void* w, const float* scale, const float* bias, void* y,
                            hipStream_t s);
// Patch-staged implicit GEMM (igemm_patch.hip): stride 1, C_in % 64 == 0,
// the tile's input patch (all channels) fits LDS next to the filter ring.
bool igemm_patch_serves(const ConvGeom& g);
int igemm_patch_num_cfgs();
bool igemm_patch_fits(const ConvGeom& g, int cfg);
int igemm_patch_choose(const ConvGeom& g);
void igemm_patch_describe(int cfg, int* BM, int* BN, int* WM, int* WN, int* WK, int* ring);
hipError_t launch_igemm_patch(const ConvGeom& g, int cfg, int epi, const void* x,
                              const void* w, const float* scale, const float* bias, void* y,
                              hipStream_t s, bool packed = false);
// Band implicit GEMM (igemm_band.hip): stride 1, C_in % 64 == 0, C_out 64
// or 128, the tile's input rows fit LDS next to the filter ring.
bool igemm_band_serves(const ConvGeom& g);
void igemm_band_describe(const ConvGeom& g, int* tile_px, int* tiles, int* lds);
hipError_t launch_igemm_band(const ConvGeom& g, int epi, const void* x, const void* w,
                             const float* scale, const float* bias, void* y, hipStream_t s);
// Bytes of tile cfg's packed filter (0: none fits 32-bit offsets), and the
// load-time pack kernel that writes it from the OHWI filter.
size_t igemm_patch_packed_bytes(const ConvGeom& g, int cfg);
hipError_t launch_pack_patch_filter(const ConvGeom& g, int cfg, const void* w, void* wp,
                                    hipStream_t s);
// Stem kernel (stem.hip): C_in = 3, 3x3, stride 2, pad 1, even W, C_out % 8 == 0
// and <= 64; one workgroup per CU walks bands of R output rows.
bool stem_serves(const ConvGeom& g);
int stem_rows(const ConvGeom& g);
bool stem_rows_ok(const ConvGeom& g, int R);
hipError_t launch_stem(const ConvGeom& g, int wg_per_cu, int R, int epi, const void* x,
                       const void* w, const float* scale, const float* bias, void* y,
                       hipStream_t s);
// Its workgroup count, and its training-mode statistics pass (C_out <= 32):
// one (count, mean, M2) triple per workgroup and channel into stats
// (stem_grid(g, stem_stats_wpc(g), R) x C_out x 3 doubles); nothing else
// stored. The statistics instance may hold more registers than the
// inference one and then runs fewer workgroups per CU (all resident).
int stem_grid(const ConvGeom& g, int wg_per_cu, int R);
bool stem_stats_serves(const ConvGeom& g);
int stem_stats_wpc(const ConvGeom& g);
hipError_t launch_stem_stats(const ConvGeom& g, int R, const void* x, const void* w,
                             double* stats, hipStream_t s);
// Tiled direct conv on MFMA (tiled_mfma.hip): K <= 32, C_out <= 32.
bool tiled_mfma_serves(const ConvGeom& g);
int tiled_mfma_rows(const ConvGeom& g);
hipError_t launch_tiled_mfma(const ConvGeom& g, int R, int epi, const void* x,
                             const void* w, const float* scale, const float* bias, void* y,
                             hipStream_t s);
bool tiled_mfma_pipe_serves(const ConvGeom& g);
hipError_t launch_tiled_mfma_pipe(const ConvGeom& g, int R, int grid, int epi,
                                  const void* x, const void* w, const float* scale,
                                  const float* bias, void* y, hipStream_t s);
hipError_t launch_bn_apply(bool f32, const void* t1, const float* scale, const float* bias, void* t2,
                           long long total, int C, hipStream_t s);
hipError_t launch_silu_apply(bool f32, const void* t2, void* y, long long total, hipStream_t s);
// Training-mode BatchNorm (train_bn.hip): per-channel batch statistics of
// t1 [M][C] into row-block partials, then scale/bias (and running estimates).
void bn_train_grid(int M, int* R, int* GX);
size_t bn_train_partial_bytes(int M, int C);
// Training mode, statistics pass of the 1x1 kernel: one (count, mean, M2)
// triple per workgroup and channel into stats (igemm_cu_stats_grid(g) x
// C_out x 3 doubles; the fixed-order merge follows); nothing else stored.
int igemm_cu_stats_grid(const ConvGeom& g);
hipError_t launch_igemm_cu_stats(const ConvGeom& g, int nwaves, int pd, const void* x,
                                 const void* w, double* stats, hipStream_t s);
size_t bn_train_chan_bytes(int G, int C);
hipError_t launch_bn_train_finalize_chan(const double* stats, int G, int M, int C,
                                         const float* gamma, const float* beta, float eps,
                                         float momentum, float* running_mean, float* running_var,
                                         float* batch_mean, float* batch_var, float* scale,
                                         float* bias, hipStream_t s);
hipError_t launch_bn_train_stats(bool f32, const void* t1, int M, int C, const float* gamma,
                                 const float* beta, float eps, float momentum,
                                 float* running_mean, float* running_var, float* batch_mean,
                                 float* batch_var, double* partial, float* scale, float* bias,
                                 hipStream_t s);
// Batched transpose src [B][R][S] -> dst [B][S][R] (layout.hip).
hipError_t launch_transpose(bool f32, const void* src, void* dst, int B, int R, int S,
                            hipStream_t s);
// Split form: y = silu(t1 * scale[c] + bias[c]) in one streaming kernel.
hipError_t launch_bn_silu_apply(bool f32, const void* t1, const float* scale, const float* bias,
                                void* y, long long total, int C, hipStream_t s);
hipError_t launch_bn_fold(const float* gamma, const float* beta, const float* mean,
                          const float* var, float eps, int C, float* scale, float* bias,
                          hipStream_t s);

}  // namespace tg
