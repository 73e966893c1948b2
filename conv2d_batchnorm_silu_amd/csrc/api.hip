// api.hip -- plan, validation, dispatch table and the C entry points declared
// in include/tg_conv_bn_silu.h.
//
// Dispatch follows "Fusing an Epilogue" (teenygrad docs), section "Three
// kernels for one operation": several kernels for one operation, chosen by
// shape with thresholds that somebody measured and wrote down, and a tile
// size derived from the layer shape and the machine's compute-unit count.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "tg_conv_bn_silu.h"
#include "tg_device.hpp"
#include "tg_internal.hpp"

using namespace tg;

namespace tg {

hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes) {
    struct Entry {
        const void* kernel;
        int device;
        size_t bytes;
    };
    static std::mutex mu;
    static std::vector<Entry> set;  // limits raised so far
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    for (Entry& en : set)
        if (en.kernel == kernel && en.device == dev) {
            if (en.bytes >= bytes) return hipSuccess;
            e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)bytes);
            if (e == hipSuccess) en.bytes = bytes;
            return e;
        }
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) set.push_back({kernel, dev, bytes});
    return e;
}

}  // namespace tg

struct tg_conv_bn_silu_plan {
    ConvGeom g;
    tg_dtype dtype;
    int kernel;      // TG_KERNEL_SCALAR / TILED / IGEMM (resolved)
    bool unfused;
    bool split;      // conv (identity epilogue) -> t1, then one bn+silu kernel
    int epi;         // fused epilogue (tg::Epilogue) from the plan's activation
    bool forced;     // kernel was requested explicitly (alignment errors instead of fallback)
    int igemm_cfg;   // index into the igemm variant table (-1: register-weights variant)
    int dma_cfg;     // >= 0: direct-to-LDS pipelined variant with this tile
    int tm_rows;     // > 0: tiled kernel runs on the matrix cores with bands of this many rows
    int tm_pipe_grid;  // > 0: ... in its persistent pipelined form with this grid
    int rw_grid;     // persistent grid of the register-weights variant
    int rw_nf, rw_cs, rw_ncw;  // its weight fragments per wave, waves per block, waves per WG
    bool rw_nt;      // non-temporal y stores in the register-weights variant
    int stream_waves;  // > 0: the streaming 1x1 kernel with this many waves per CU
    int xdma;        // ... staging x through LDS with this prefetch depth (0: off)
    int cu_waves;    // > 0: one-workgroup-per-CU variant with this many wavefronts
    int cu_pd;       // ... and this input prefetch depth
    bool band;       // band implicit GEMM (all output channels of a pixel band per workgroup)
    int patch_cfg;   // >= 0: patch-staged implicit GEMM with this tile
    int stem_wpc;    // > 0: stem kernel with this many workgroups per CU
    int stem_rows;   // ... and bands of this many output rows
    TiledCfg tiled;
    size_t ws_bytes;  // unfused and split only
};

namespace {

// MI355X: 256 compute units in 8 XCDs. Tile choice is a function of the shape
// and of this count only, so plans are reproducible on any host.
const int kCUs = 256;

// Rates the cost model uses, per clock at 2.4 GHz. The microbenchmarks in
// peaks.hip (profiles/peaks_mi355x.md) measure on MI355X: 16x16x32 f16 MFMA
// 922 (one wave per SIMD) to 961 (two) FLOP per clock per SIMD, i.e.
// 2.27-2.36 PFLOP/s, of which the model assumes 94%; conflict-free
// ds_read_b128 146 (4 waves) to 250 (8 waves) bytes per clock per CU.
const double kClock = 2.4e9;
const double kMfmaFlopPerClkSimd = 871.0;  // 2.14 PFLOP/s on the whole chip
const double kLdsBytesPerClkCu = 213.0;     // ds_read_b128 at 6-8 waves per CU
const double kHbmBytesPerSec = 5.0e12;      // mixed read/write streaming
const double kL2FillBytesPerClkCu = 64.0;

// Kernel-variant overrides for measurement and tests
// (tg_conv_bn_silu_create_tuned). Each field is -1 unless the caller's tuning
// string sets it; plans never read the process environment.
struct Tuning {
    int cu = -1, cu_pd = -1, igemm_rw = -1, rw_nf = -1, rw_cs = -1, rw_ncw = -1;
    int rw_wg_per_cu = -1, nt = -1, stream = -1, xdma = -1, igemm_patch = -1;
    int patch_cfg = -1, igemm_dma = -1, dma_cfg = -1, igemm_cfg = -1, stem = -1;
    int stem_rows = -1, tiled_mfma = -1, tm_rows = -1, tm_pipe = -1, tm_wg_per_cu = -1;
    int band = -1;
};

struct TuningKey {
    const char* name;
    int Tuning::*field;
};
const TuningKey kTuningKeys[] = {
    {"cu", &Tuning::cu}, {"cu_pd", &Tuning::cu_pd}, {"igemm_rw", &Tuning::igemm_rw},
    {"rw_nf", &Tuning::rw_nf}, {"rw_cs", &Tuning::rw_cs}, {"rw_ncw", &Tuning::rw_ncw},
    {"rw_wg_per_cu", &Tuning::rw_wg_per_cu}, {"nt", &Tuning::nt}, {"stream", &Tuning::stream},
    {"xdma", &Tuning::xdma}, {"igemm_patch", &Tuning::igemm_patch},
    {"patch_cfg", &Tuning::patch_cfg}, {"igemm_dma", &Tuning::igemm_dma},
    {"dma_cfg", &Tuning::dma_cfg}, {"igemm_cfg", &Tuning::igemm_cfg}, {"stem", &Tuning::stem},
    {"stem_rows", &Tuning::stem_rows}, {"tiled_mfma", &Tuning::tiled_mfma},
    {"tm_rows", &Tuning::tm_rows}, {"tm_pipe", &Tuning::tm_pipe},
    {"tm_wg_per_cu", &Tuning::tm_wg_per_cu}, {"band", &Tuning::band},
};

// "key=value[,key=value...]" with known keys and values in [0, 2^20); NULL or
// "" is no override. Returns false for anything else.
bool parse_tuning(const char* s, Tuning* t) {
    *t = Tuning();
    if (!s) return true;
    while (*s) {
        const char* eq = strchr(s, '=');
        if (!eq) return false;
        const size_t klen = (size_t)(eq - s);
        const TuningKey* key = nullptr;
        for (const TuningKey& k : kTuningKeys)
            if (strlen(k.name) == klen && strncmp(k.name, s, klen) == 0) key = &k;
        if (!key) return false;
        const char* v = eq + 1;
        long val = 0;
        int digits = 0;
        while (*v >= '0' && *v <= '9' && digits < 8) {
            val = val * 10 + (*v - '0');
            ++v;
            ++digits;
        }
        if (digits == 0 || val >= (1L << 20) || (*v != ',' && *v != '\0')) return false;
        if (*v == ',' && v[1] == '\0') return false;  // trailing comma
        t->*(key->field) = (int)val;
        s = *v == ',' ? v + 1 : v;
    }
    return true;
}

// The override if given, else the default.
int tuned(int v, int dflt) { return v >= 0 ? v : dflt; }

// An enum argument as the int the caller passed. C callers may pass any int
// where the header names an enum; reading such a value through the C++ enum
// type is undefined when it lies outside the enum's range, so entry points
// take the bits as an int first and validate that.
template <class E>
int ival(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "enum arguments are int-sized");
    int v;
    memcpy(&v, &e, sizeof(v));
    return v;
}

long long out_extent(long long in, long long k, long long stride, long long pad) {
    if (in + 2 * pad < k) return 0;
    return (in + 2 * pad - k) / stride + 1;
}

tg_status make_geom(int N, int H, int W, int C_in, int C_out, int kh, int kw, int stride, int pad,
                    ConvGeom* g) {
    if (N < 1 || H < 1 || W < 1 || C_in < 1 || C_out < 1 || kh < 1 || kw < 1 || stride < 1 ||
        pad < 0)
        return TG_ERR_INVALID_ARGUMENT;
    long long P = out_extent(H, kh, stride, pad), Q = out_extent(W, kw, stride, pad);
    if (P < 1 || Q < 1) return TG_ERR_INVALID_ARGUMENT;
    const long long lim = (1LL << 31) - 1;
    long long nx = (long long)N * H * W * C_in;
    long long nw = (long long)C_out * kh * kw * C_in;
    long long ny = (long long)N * P * Q * C_out;
    if (nx > lim || nw > lim || ny > lim) return TG_ERR_UNSUPPORTED;
    // Padded extents and strided offsets stay far below 2^31 as well.
    if ((long long)H + 2LL * pad > lim / 4 || (long long)W + 2LL * pad > lim / 4)
        return TG_ERR_UNSUPPORTED;
    g->N = N; g->H = H; g->W = W; g->C_in = C_in; g->C_out = C_out;
    g->kh = kh; g->kw = kw; g->stride = stride; g->pad = pad;
    g->P = (int)P; g->Q = (int)Q;
    g->M = (int)(N * P * Q);
    g->K = kh * kw * C_in;
    g->out8 = 0;
    g->res = nullptr;
    return TG_OK;
}

bool igemm_serves(const ConvGeom& g, tg_dtype dt) { return dt == TG_F16 && g.C_in % 8 == 0; }

bool tiled_serves(const ConvGeom& g, tg_dtype dt, TiledCfg* c) {
    TiledCfg tmp;
    return dt == TG_F16 && tiled_plan(g, c ? c : &tmp);
}

// Estimated time of an igemm variant: the busiest CU's MFMA work (scaled up
// when the wave tile reads LDS faster than LDS delivers) against the memory
// time (compulsory HBM bytes plus the L2 -> LDS operand fill of every tile).
double igemm_cost(const ConvGeom& g, const IgemmCfg& c) {
    long long tiles_m = (g.M + c.BM - 1) / c.BM, tiles_n = (g.C_out + c.BN - 1) / c.BN;
    long long tiles = tiles_m * tiles_n;
    long long kpad = (g.K + c.BK - 1) / c.BK * c.BK;
    long long per_cu = (tiles + kCUs - 1) / kCUs;
    int FM = c.BM / c.WM / 16, FN = c.BN / c.WN / 16;
    double mfma_clk = 16384.0 / kMfmaFlopPerClkSimd;  // one 16x16x32 instruction
    double lds_need = 4.0 * (FM + FN) * 1024.0 / (FM * FN * mfma_clk);  // B/clk per CU
    double lds_factor = lds_need > kLdsBytesPerClkCu ? lds_need / kLdsBytesPerClkCu : 1.0;
    double t_mfma = per_cu * (double)c.BM * c.BN * kpad * 2.0 /
                    (4.0 * kMfmaFlopPerClkSimd * kClock) * lds_factor;
    double hbm = 2.0 * ((double)g.N * g.H * g.W * g.C_in + (double)g.M * g.C_out +
                        (double)g.C_out * g.K);
    double fill = (double)tiles * (c.BM + c.BN) * kpad * 2.0;
    double t_mem = hbm / kHbmBytesPerSec + fill / (kCUs * kL2FillBytesPerClkCu * kClock);
    return t_mfma > t_mem ? t_mfma : t_mem;
}

// Estimated time of a direct-to-LDS igemm tile: one workgroup per CU at a
// time, so the busiest CU runs ceil(tiles / CUs) tiles back to back; the
// wave tile's LDS read rate scales the MFMA time when it exceeds LDS speed.
double igemm_dma_cost(const ConvGeom& g, const IgemmCfg& c) {
    long long tiles = (long long)((g.M + c.BM - 1) / c.BM) * ((g.C_out + c.BN - 1) / c.BN);
    long long per_cu = (tiles + kCUs - 1) / kCUs;
    int FM = c.BM / c.WM / 16, FN = c.BN / c.WN / 16;
    double mfma_clk = 16384.0 / kMfmaFlopPerClkSimd;
    double lds_need = 4.0 * (FM + FN) * 1024.0 / (FM * FN * mfma_clk);
    double lds_factor = lds_need > kLdsBytesPerClkCu ? lds_need / kLdsBytesPerClkCu : 1.0;
    // Two K-groups (two waves per SIMD) overlap fragment reads with MFMAs:
    // 12-14% faster on the 3x3 and 7x7 layers measured on MI355X.
    double overlap = c.WK == 2 ? 0.88 : 1.0;
    return per_cu * (double)c.BM * c.BN * g.K * lds_factor * overlap;
}

int choose_igemm_dma_cfg(const ConvGeom& g, const Tuning& tu) {
    int forced = tu.dma_cfg;
    if (forced >= 0 && forced < igemm_dma_num_cfgs()) return forced;
    int best = 0;
    double best_cost = 1e300;
    for (int i = 0; i < igemm_dma_num_cfgs(); ++i) {
        double c = igemm_dma_cost(g, igemm_dma_cfg(i));
        if (c < best_cost) { best = i; best_cost = c; }
    }
    return best;
}

int choose_igemm_cfg(const ConvGeom& g, const Tuning& tu) {
    int forced = tu.igemm_cfg;
    if (forced >= 0 && forced < igemm_num_cfgs()) return forced;
    int best = 0;
    double best_cost = 1e300;
    for (int i = 0; i < igemm_num_cfgs(); ++i) {
        const IgemmCfg& c = igemm_cfg(i);
        double cost = igemm_cost(g, c);
        // Ties (within 2%) go to the wider channel tile: fewer re-reads of x.
        if (cost < best_cost * 0.98 ||
            (cost < best_cost * 1.02 && c.BN > igemm_cfg(best).BN)) {
            best = i;
            best_cost = cost < best_cost ? cost : best_cost;
        }
    }
    return best;
}

tg_kernel dispatch(const ConvGeom& g, tg_dtype dt, tg_dispatch table) {
    if (table == TG_DISPATCH_PAGES) {
        // The page's table: GEMM for 1x1 convolutions with at least 32 output
        // channels, tiled above 16 output channels, scalar otherwise. A kernel
        // that cannot serve the shape passes it to the next rule.
        if (g.kh == 1 && g.kw == 1 && g.C_out >= 32 && igemm_serves(g, dt)) return TG_KERNEL_IGEMM;
        if (g.C_out > 16 && tiled_serves(g, dt, nullptr)) return TG_KERNEL_TILED;
        return TG_KERNEL_SCALAR;
    }
    // MI355X table, from timing every kernel that serves a shape over k in
    // {1,3,5,7}, stride {1,2}, C_in {3,16,64,128}, C_out {8..256} at 10^5
    // output pixels (sweep_dispatch.py; MI355X, gfx950, ROCm 7.2):
    //  * C_in % 8 == 0: the implicit GEMM wins at every C_out (2.7-78x over
    //    the tiled and scalar kernels from C_out 8 on), except 1x1 layers
    //    with K < 32 and C_out <= 32, where the MFMA tiled kernel is 5-15%
    //    faster;
    //  * otherwise (RGB input): tiled wherever it fits, except 1x1 layers
    //    beyond the MFMA tiled kernel's C_out <= 32, where the VALU tiled
    //    kernel loses to the scalar one (1.3-1.75x); scalar past C_out 64.
    if (dt == TG_F32) return TG_KERNEL_SCALAR;
    if (igemm_serves(g, dt)) {
        if (g.K < 32 && tiled_mfma_serves(g) && tiled_serves(g, dt, nullptr)) return TG_KERNEL_TILED;
        return TG_KERNEL_IGEMM;
    }
    if (tiled_serves(g, dt, nullptr)) {
        if (g.kh * g.kw == 1 && !tiled_mfma_serves(g)) return TG_KERNEL_SCALAR;
        return TG_KERNEL_TILED;
    }
    return TG_KERNEL_SCALAR;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

tg_status create_impl(tg_conv_bn_silu_plan** out, int N, int H, int W, int C_in, int C_out, int kh,
                      int kw, int stride, int pad, int dtype_v, int kernel_v, int table_v,
                      int act_v = TG_ACT_SILU, bool out_fp8 = false,
                      const char* tuning = nullptr) {
    if (!out) return TG_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    Tuning tu;
    if (!parse_tuning(tuning, &tu)) return TG_ERR_INVALID_ARGUMENT;
    ConvGeom g;
    tg_status st = make_geom(N, H, W, C_in, C_out, kh, kw, stride, pad, &g);
    if (st != TG_OK) return st;
    if (dtype_v != TG_F16 && dtype_v != TG_F32) return TG_ERR_UNSUPPORTED;
    if (table_v != TG_DISPATCH_MI355X && table_v != TG_DISPATCH_PAGES) return TG_ERR_UNSUPPORTED;
    if (act_v < TG_ACT_SILU || act_v > TG_ACT_NONE) return TG_ERR_UNSUPPORTED;
    const tg_dtype dtype = (tg_dtype)dtype_v;
    const tg_dispatch table = (tg_dispatch)table_v;
    const tg_activation act = (tg_activation)act_v;
    int kv = kernel_v;
    bool unfused = (kv & TG_UNFUSED) != 0;
    bool split = (kv & TG_SPLIT) != 0;
    if (unfused && split) return TG_ERR_UNSUPPORTED;
    int epi;
    switch (act) {
        case TG_ACT_SILU: epi = EPI_FUSED; break;
        case TG_ACT_RELU: epi = EPI_RELU; break;
        case TG_ACT_GELU: epi = EPI_GELU; break;
        case TG_ACT_NONE: epi = EPI_BN; break;
        default: return TG_ERR_UNSUPPORTED;
    }
    // The baselines' streaming kernels apply BatchNorm and SiLU only, and
    // write y in the input dtype.
    if ((unfused || split) && (epi != EPI_FUSED || out_fp8)) return TG_ERR_UNSUPPORTED;
    if (out_fp8 && dtype != TG_F16) return TG_ERR_UNSUPPORTED;
    int base = kv & ~(TG_UNFUSED | TG_SPLIT);
    if (base < TG_KERNEL_AUTO || base > TG_KERNEL_IGEMM) return TG_ERR_UNSUPPORTED;

    tg_conv_bn_silu_plan p;
    memset(&p, 0, sizeof(p));
    p.g = g;
    p.dtype = dtype;
    p.unfused = unfused;
    p.split = split;
    p.epi = epi;
    p.g.out8 = out_fp8 ? 1 : 0;
    p.forced = base != TG_KERNEL_AUTO;
    p.dma_cfg = -1;
    p.patch_cfg = -1;
    p.kernel = p.forced ? base : (int)dispatch(g, dtype, table);
    if (p.kernel == TG_KERNEL_IGEMM) {
        if (!igemm_serves(g, dtype)) return TG_ERR_UNSUPPORTED;
        if (igemm_rw_serves(g) && tuned(tu.igemm_rw, 1) != 0 && tu.igemm_cfg < 0) {
            p.igemm_cfg = -1;
            igemm_rw_choose(g, &p.rw_nf, &p.rw_cs, &p.rw_ncw);
            p.rw_nf = tuned(tu.rw_nf, p.rw_nf);
            p.rw_cs = tuned(tu.rw_cs, p.rw_cs);
            p.rw_ncw = tuned(tu.rw_ncw, p.rw_ncw);
            if (!igemm_rw_valid(g, p.rw_nf, p.rw_cs, p.rw_ncw))  // override does not fit
                igemm_rw_choose(g, &p.rw_nf, &p.rw_cs, &p.rw_ncw);
            p.rw_grid = igemm_rw_grid(g, kCUs * (tu.rw_wg_per_cu > 0 ? tu.rw_wg_per_cu : 1));
            p.rw_nt = tuned(tu.nt, 1) != 0;
            p.stream_waves = tu.stream > 0 ? tu.stream : 0;
            p.xdma = tuned(tu.xdma, 0);
            // cu: wavefronts per 64-channel slice of the one-workgroup-per-CU
            // kernel (0 disables it); cu_pd: input blocks in flight per
            // wavefront (1..3). 3 and 3 (12 wavefronts for 256 channels, three
            // blocks ahead) measured best on MI355X for the 1x1 C_in=64 layer
            // with settled clocks (12.9 us mean over four runs against 13.5 us
            // two blocks ahead, and a tighter spread). The register-weights
            // kernel stays the fallback for BatchNorm vectors that are not
            // 16-byte aligned.
            if (igemm_cu_serves(g) && tuned(tu.cu, 3) > 0) {
                p.cu_waves = igemm_cu_waves(g, tuned(tu.cu, 3));
                p.cu_pd = tuned(tu.cu_pd, 3);
                if (p.cu_pd < 1 || p.cu_pd > 3) return TG_ERR_INVALID_ARGUMENT;
            }
        } else if (igemm_band_serves(g) && tuned(tu.band, 0) != 0 && tu.igemm_cfg < 0 &&
                   // Opt-in: on the 3x3 and 7x7 layers it runs level with
                   // (3x3) or 8% behind (7x7) the patch-staged kernel below.
                   tu.patch_cfg < 0 && tu.dma_cfg < 0) {
            p.igemm_cfg = 0;
            p.band = true;
        } else if (igemm_patch_serves(g) && tuned(tu.igemm_patch, 1) != 0 &&
                   tu.igemm_cfg < 0) {
            // patch_cfg forces a tile (if it fits this shape's LDS need).
            p.igemm_cfg = 0;
            int forced = tu.patch_cfg;
            p.patch_cfg = igemm_patch_fits(g, forced) ? forced : igemm_patch_choose(g);
        } else if (igemm_dma_serves(g) && tuned(tu.igemm_dma, 1) != 0 && tu.igemm_cfg < 0) {
            p.igemm_cfg = 0;
            p.dma_cfg = choose_igemm_dma_cfg(g, tu);
        } else {
            p.igemm_cfg = choose_igemm_cfg(g, tu);
        }
    } else if (p.kernel == TG_KERNEL_TILED) {
        if (!tiled_serves(g, dtype, &p.tiled)) return TG_ERR_UNSUPPORTED;
        // stem: workgroups per CU of the stem kernel (0 disables it);
        // stem_rows: output rows per band.
        if (stem_serves(g) && tuned(tu.stem, 3) > 0) {
            p.stem_wpc = tuned(tu.stem, 3);
            p.stem_rows = tuned(tu.stem_rows, stem_rows(g));
            if (!stem_rows_ok(g, p.stem_rows)) p.stem_rows = stem_rows(g);
        }
        if (tiled_mfma_serves(g) && tuned(tu.tiled_mfma, 1) != 0) {
            p.tm_rows = tu.tm_rows > 0 ? tu.tm_rows : tiled_mfma_rows(g);
            if (tiled_mfma_pipe_serves(g) && tuned(tu.tm_pipe, 1) != 0) {
                p.tm_rows = tu.tm_rows > 0 ? tu.tm_rows : 2;
                p.tm_pipe_grid = kCUs * (tu.tm_wg_per_cu > 0 ? tu.tm_wg_per_cu : 4);
            }
        }
    }
    size_t ysz = (size_t)g.M * g.C_out * (dtype == TG_F16 ? 2 : 4);
    p.ws_bytes = unfused ? 2 * round256(ysz) : (split ? round256(ysz) : 0);

    tg_conv_bn_silu_plan* h = new (std::nothrow) tg_conv_bn_silu_plan(p);
    if (!h) return TG_ERR_UNSUPPORTED;
    *out = h;
    return TG_OK;
}

// Launch the plan's conv kernel (or `kernel`, after an alignment fallback)
// writing `out`, with epilogue `epi` (tg::Epilogue).
hipError_t launch_conv(const tg_conv_bn_silu_plan* plan, const ConvGeom& g, int kernel, int epi,
                       const void* x,
                       const void* w, const float* bn_scale, const float* bn_bias, void* conv_out,
                       hipStream_t s) {
    const bool f32 = plan->dtype == TG_F32;
    hipError_t e;
    switch (kernel) {
        case TG_KERNEL_IGEMM:
            if (plan->cu_waves > 0 && aligned16(bn_scale) && aligned16(bn_bias))
                e = launch_igemm_cu(g, plan->cu_waves, plan->cu_pd, plan->rw_nt, epi, x, w,
                                    bn_scale, bn_bias, conv_out, s);
            else if (plan->igemm_cfg < 0 && plan->stream_waves > 0 &&
                     (epi == EPI_FUSED || epi == EPI_IDENTITY))
                e = launch_igemm_stream(g, plan->stream_waves, plan->xdma, plan->rw_nt, epi, x, w,
                                        bn_scale, bn_bias, conv_out, s);
            else if (plan->band)
                e = launch_igemm_band(g, epi, x, w, bn_scale, bn_bias, conv_out, s);
            else if (plan->patch_cfg >= 0)
                e = launch_igemm_patch(g, plan->patch_cfg, epi, x, w, bn_scale, bn_bias,
                                       conv_out, s);
            else if (plan->dma_cfg >= 0)
                e = launch_igemm_dma(g, plan->dma_cfg, epi, x, w, bn_scale, bn_bias, conv_out,
                                     s);
            else if (plan->igemm_cfg < 0)
                e = launch_igemm_rw(g, plan->rw_grid, plan->rw_nf, plan->rw_cs, plan->rw_ncw,
                                    plan->rw_nt, epi, x, w, bn_scale, bn_bias, conv_out, s);
            else
                e = launch_igemm(g, plan->igemm_cfg, epi, x, w, bn_scale, bn_bias, conv_out,
                                 s);
            break;
        case TG_KERNEL_TILED:
            if (plan->stem_wpc > 0)
                e = launch_stem(g, plan->stem_wpc, plan->stem_rows, epi, x, w, bn_scale, bn_bias,
                                conv_out, s);
            else if (plan->tm_pipe_grid > 0)
                e = launch_tiled_mfma_pipe(g, plan->tm_rows, plan->tm_pipe_grid, epi, x, w,
                                           bn_scale, bn_bias, conv_out, s);
            else if (plan->tm_rows > 0)
                e = launch_tiled_mfma(g, plan->tm_rows, epi, x, w, bn_scale, bn_bias,
                                      conv_out, s);
            else
                e = launch_tiled(g, plan->tiled, epi, x, w, bn_scale, bn_bias, conv_out, s);
            break;
        default:
            e = launch_scalar(g, f32, epi, x, w, bn_scale, bn_bias, conv_out, s);
            break;
    }
    return e;
}

// Device memory for tg_conv_bn_silu_train_run_static: one copy of this array
// per GPU, at its own address on each. In host code `scratch` names a
// host-side stand-in, never the device memory: kernels and copies take the
// address from static_scratch().
static __device__ __align__(256) unsigned char scratch[TG_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device; written once under g_scratch_mu

// The array's device address on the current device, looked up (under the
// lock) at the first call there.
tg_status static_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return TG_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return TG_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TG_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TG_OK;
}

// Training mode: the 1x1 and stem layers take their statistics from a conv
// pass that stores nothing and then run the fused kernel; the other layers
// keep t1 in y (the BatchNorm+SiLU pass then works on y in place). Workspace: [scale
// fp32 [C]][bias fp32 [C]][statistics partials: fp64 row-block sums, or the
// 1x1 kernel's per-workgroup triples], each piece 256-byte aligned.
struct TrainWs {
    size_t scale, bias, partial, total;
};
TrainWs train_ws(const tg_conv_bn_silu_plan* plan) {
    const ConvGeom& g = plan->g;
    const size_t vec = round256((size_t)g.C_out * 4);
    size_t part = bn_train_partial_bytes(g.M, g.C_out);
    if (igemm_cu_serves(g)) {
        const size_t chan = bn_train_chan_bytes(igemm_cu_stats_grid(g), g.C_out);
        if (chan > part) part = chan;
    }
    if (plan->stem_wpc > 0 && stem_stats_serves(g)) {
        const size_t chan =
            bn_train_chan_bytes(stem_grid(g, stem_stats_wpc(g), plan->stem_rows), g.C_out);
        if (chan > part) part = chan;
    }
    TrainWs t;
    t.scale = 0;
    t.bias = vec;
    t.partial = 2 * vec;
    t.total = t.partial + round256(part);
    return t;
}

// Argument checks shared by the training entry points.
tg_status train_check(const tg_conv_bn_silu_plan* plan, const void* x, const void* w,
                      const float* gamma, const float* beta, float eps, float momentum,
                      const float* running_mean, const float* running_var, const void* y) {
    if (!plan || !x || !w || !gamma || !beta || !y) return TG_ERR_INVALID_ARGUMENT;
    if ((running_mean == nullptr) != (running_var == nullptr)) return TG_ERR_INVALID_ARGUMENT;
    if (!(eps >= 0.0f) || !(momentum >= 0.0f && momentum <= 1.0f)) return TG_ERR_INVALID_ARGUMENT;
    if (plan->g.M < 2) return TG_ERR_INVALID_ARGUMENT;  // batch statistics need two values per channel
    if (plan->epi != EPI_FUSED || plan->g.out8) return TG_ERR_UNSUPPORTED;  // SiLU, y in dtype
    return TG_OK;
}

// The training passes on stream s, with scale, bias and the statistics
// partials at ws (train_ws layout, device memory the caller provides).
tg_status train_core(const tg_conv_bn_silu_plan* plan, const void* x, const void* w,
                     const float* gamma, const float* beta, float eps, float momentum,
                     float* running_mean, float* running_var, float* batch_mean,
                     float* batch_var, void* y, char* ws, hipStream_t s) {
    const ConvGeom& g = plan->g;
    const TrainWs L = train_ws(plan);
    const bool f32 = plan->dtype == TG_F32;
    int kernel = plan->kernel;
    if (kernel != TG_KERNEL_SCALAR &&
        !(aligned16(x) && aligned16(w) && aligned16(y) && aligned16(ws))) {
        if (plan->forced) return TG_ERR_ALIGNMENT;
        kernel = TG_KERNEL_SCALAR;
    }
    float* scale = (float*)(ws + L.scale);
    float* bias = (float*)(ws + L.bias);
    double* partial = (double*)(ws + L.partial);
    hipError_t e;
    if (kernel == TG_KERNEL_IGEMM && plan->cu_waves > 0 && !plan->unfused && !plan->split && !f32) {
        // The 1x1 layer is bound by HBM, not by its arithmetic: its
        // statistics come from a pass of the conv that reads x and stores
        // nothing (at most 12 waves: the statistics take registers), and the
        // fused kernel then computes the conv again with the batch
        // statistics folded into scale and bias. That reads x twice instead
        // of writing t1 and reading and writing it again, and y is the
        // BatchNorm+SiLU of the fp32 accumulators, as in inference.
        const int ng = g.C_out / 64;
        int nw = plan->cu_waves;
        if (nw > 12) nw = 12 / ng * ng;
        e = launch_igemm_cu_stats(g, nw, plan->cu_pd, x, w, partial, s);
        if (e != hipSuccess) return TG_ERR_HIP;
        e = launch_bn_train_finalize_chan(partial, igemm_cu_stats_grid(g), g.M, g.C_out, gamma,
                                          beta, eps, momentum, running_mean, running_var,
                                          batch_mean, batch_var, scale, bias, s);
        if (e != hipSuccess) return TG_ERR_HIP;
        e = launch_conv(plan, g, kernel, plan->epi, x, w, scale, bias, y, s);
        return e == hipSuccess ? TG_OK : TG_ERR_HIP;
    } else if (kernel == TG_KERNEL_TILED && plan->stem_wpc > 0 && stem_stats_serves(g) &&
               !plan->unfused && !plan->split && !f32) {
        // The stem (HBM-bound as well): the same two passes with the stem
        // kernel's statistics instance.
        e = launch_stem_stats(g, plan->stem_rows, x, w, partial, s);
        if (e != hipSuccess) return TG_ERR_HIP;
        e = launch_bn_train_finalize_chan(partial, stem_grid(g, stem_stats_wpc(g), plan->stem_rows),
                                          g.M, g.C_out, gamma, beta, eps, momentum, running_mean,
                                          running_var, batch_mean, batch_var, scale, bias, s);
        if (e != hipSuccess) return TG_ERR_HIP;
        e = launch_conv(plan, g, kernel, plan->epi, x, w, scale, bias, y, s);
        return e == hipSuccess ? TG_OK : TG_ERR_HIP;
    } else {
        // 1. conv -> t1 in y (identity epilogue: scale/bias are not read)
        e = launch_conv(plan, g, kernel, EPI_IDENTITY, x, w, scale, bias, y, s);
        if (e != hipSuccess) return TG_ERR_HIP;
        // 2-3. batch statistics -> scale, bias, running estimates
        e = launch_bn_train_stats(f32, y, g.M, g.C_out, gamma, beta, eps, momentum, running_mean,
                                  running_var, batch_mean, batch_var, partial, scale, bias, s);
    }
    if (e != hipSuccess) return TG_ERR_HIP;
    // 4. BatchNorm + SiLU on y in place
    e = launch_bn_silu_apply(f32, y, scale, bias, y, (long long)g.M * g.C_out, g.C_out, s);
    return e == hipSuccess ? TG_OK : TG_ERR_HIP;
}

}  // namespace

extern "C" {

tg_status tg_conv_bn_silu_create(tg_conv_bn_silu_plan** out, int N, int H, int W, int C_in,
                                 int C_out, int kh, int kw, int stride, int pad, tg_dtype dtype,
                                 tg_kernel kernel) {
    return create_impl(out, N, H, W, C_in, C_out, kh, kw, stride, pad, ival(dtype), ival(kernel),
                       TG_DISPATCH_MI355X);
}

tg_status tg_conv_bn_silu_create_with_table(tg_conv_bn_silu_plan** out, int N, int H, int W,
                                            int C_in, int C_out, int kh, int kw, int stride,
                                            int pad, tg_dtype dtype, tg_kernel kernel,
                                            tg_dispatch table) {
    return create_impl(out, N, H, W, C_in, C_out, kh, kw, stride, pad, ival(dtype), ival(kernel),
                       ival(table));
}

tg_status tg_conv_bn_act_create(tg_conv_bn_silu_plan** out, int N, int H, int W, int C_in,
                                int C_out, int kh, int kw, int stride, int pad, tg_dtype dtype,
                                tg_kernel kernel, tg_activation act) {
    return create_impl(out, N, H, W, C_in, C_out, kh, kw, stride, pad, ival(dtype), ival(kernel),
                       TG_DISPATCH_MI355X, ival(act));
}

// y in the input dtype or fp8; anything else is TG_ERR_UNSUPPORTED.
static tg_status create_out(tg_conv_bn_silu_plan** out, int N, int H, int W, int C_in, int C_out,
                            int kh, int kw, int stride, int pad, int dtype, int kernel, int act,
                            int y_dtype, const char* tuning) {
    if (y_dtype != dtype && y_dtype != TG_F8_E4M3) {
        if (out) *out = nullptr;
        return TG_ERR_UNSUPPORTED;
    }
    return create_impl(out, N, H, W, C_in, C_out, kh, kw, stride, pad, dtype, kernel,
                       TG_DISPATCH_MI355X, act, y_dtype == TG_F8_E4M3,
                       tuning);
}

tg_status tg_conv_bn_act_create_out(tg_conv_bn_silu_plan** out, int N, int H, int W, int C_in,
                                    int C_out, int kh, int kw, int stride, int pad,
                                    tg_dtype dtype, tg_kernel kernel, tg_activation act,
                                    tg_dtype y_dtype) {
    return create_out(out, N, H, W, C_in, C_out, kh, kw, stride, pad, ival(dtype), ival(kernel),
                      ival(act), ival(y_dtype), nullptr);
}

tg_status tg_conv_bn_silu_create_tuned(tg_conv_bn_silu_plan** out, int N, int H, int W, int C_in,
                                       int C_out, int kh, int kw, int stride, int pad,
                                       tg_dtype dtype, tg_kernel kernel, tg_activation act,
                                       tg_dtype y_dtype, const char* tuning) {
    return create_out(out, N, H, W, C_in, C_out, kh, kw, stride, pad, ival(dtype), ival(kernel),
                      ival(act), ival(y_dtype), tuning);
}

tg_status tg_conv_bn_silu_destroy(tg_conv_bn_silu_plan* plan) {
    delete plan;
    return TG_OK;
}

static tg_status run_impl(const tg_conv_bn_silu_plan* plan, const void* x, const void* w,
                          const float* bn_scale, const float* bn_bias, const void* residual,
                          void* y, void* workspace, size_t workspace_bytes, void* stream) {
    if (!plan || !x || !w || !bn_scale || !bn_bias || !y) return TG_ERR_INVALID_ARGUMENT;
    const ConvGeom& g = plan->g;
    hipStream_t s = (hipStream_t)stream;
    bool f32 = plan->dtype == TG_F32;
    int kernel = plan->kernel;
    if (kernel != TG_KERNEL_SCALAR &&
        !(aligned16(x) && aligned16(w) && aligned16(y) && (!residual || aligned16(residual)))) {
        if (plan->forced) return TG_ERR_ALIGNMENT;
        kernel = TG_KERNEL_SCALAR;
    }
    void* conv_out = y;
    void* t2 = nullptr;
    if (plan->unfused || plan->split) {
        if (!workspace || workspace_bytes < plan->ws_bytes) return TG_ERR_WORKSPACE;
        size_t ysz = (size_t)g.M * g.C_out * (f32 ? 4 : 2);
        conv_out = workspace;
        if (plan->unfused) t2 = (char*)workspace + round256(ysz);
        if (kernel != TG_KERNEL_SCALAR && !aligned16(workspace)) {
            if (plan->forced) return TG_ERR_ALIGNMENT;
            kernel = TG_KERNEL_SCALAR;
        }
    }
    const int epi = plan->unfused || plan->split ? EPI_IDENTITY : plan->epi;
    ConvGeom gr = g;
    gr.res = residual;
    hipError_t e = launch_conv(plan, gr, kernel, epi, x, w, bn_scale, bn_bias, conv_out, s);
    if (e != hipSuccess) return TG_ERR_HIP;
    if (plan->unfused) {
        long long total = (long long)g.M * g.C_out;
        e = launch_bn_apply(f32, conv_out, bn_scale, bn_bias, t2, total, g.C_out, s);
        if (e != hipSuccess) return TG_ERR_HIP;
        e = launch_silu_apply(f32, t2, y, total, s);
        if (e != hipSuccess) return TG_ERR_HIP;
    } else if (plan->split) {
        long long total = (long long)g.M * g.C_out;
        e = launch_bn_silu_apply(f32, conv_out, bn_scale, bn_bias, y, total, g.C_out, s);
        if (e != hipSuccess) return TG_ERR_HIP;
    }
    return TG_OK;
}

tg_status tg_conv_bn_silu_train_workspace(const tg_conv_bn_silu_plan* plan, size_t* bytes) {
    if (!plan || !bytes) return TG_ERR_INVALID_ARGUMENT;
    *bytes = train_ws(plan).total;
    return TG_OK;
}

tg_status tg_conv_bn_silu_train_run_static(const tg_conv_bn_silu_plan* plan, const void* x,
                                           const void* w, const float* gamma, const float* beta,
                                           float eps, float momentum, float* running_mean,
                                           float* running_var, float* batch_mean,
                                           float* batch_var, void* y, void* stream) {
    tg_status st = train_check(plan, x, w, gamma, beta, eps, momentum, running_mean, running_var, y);
    if (st != TG_OK) return st;
    if (train_ws(plan).total > (size_t)TG_STATIC_SCRATCH_BYTES) return TG_ERR_UNSUPPORTED;
    void* ws = nullptr;
    st = static_scratch(&ws);
    if (st != TG_OK) return st;
    return train_core(plan, x, w, gamma, beta, eps, momentum, running_mean, running_var,
                      batch_mean, batch_var, y, (char*)ws, (hipStream_t)stream);
}

tg_status tg_conv_bn_silu_train_run(const tg_conv_bn_silu_plan* plan, const void* x, const void* w,
                                    const float* gamma, const float* beta, float eps,
                                    float momentum, float* running_mean, float* running_var,
                                    float* batch_mean, float* batch_var, void* y, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    tg_status st = train_check(plan, x, w, gamma, beta, eps, momentum, running_mean, running_var, y);
    if (st != TG_OK) return st;
    if (!workspace || workspace_bytes < train_ws(plan).total) return TG_ERR_WORKSPACE;
    return train_core(plan, x, w, gamma, beta, eps, momentum, running_mean, running_var,
                      batch_mean, batch_var, y, (char*)workspace, (hipStream_t)stream);
}

static tg_status transpose_entry(const void* src, void* dst, long long B, long long R,
                                 long long S, int dtype, void* stream) {
    if (!src || !dst || src == dst || B < 1 || R < 1 || S < 1) return TG_ERR_INVALID_ARGUMENT;
    if (dtype != TG_F16 && dtype != TG_F32) return TG_ERR_UNSUPPORTED;
    if (B * R * S >= (1LL << 31)) return TG_ERR_UNSUPPORTED;
    hipError_t e = launch_transpose(dtype == TG_F32, src, dst, (int)B, (int)R, (int)S,
                                    (hipStream_t)stream);
    return e == hipSuccess ? TG_OK : TG_ERR_HIP;
}

tg_status tg_nchw_to_nhwc(const void* src, void* dst, int N, int C, int H, int W,
                          tg_dtype dtype, void* stream) {
    if (N < 1 || C < 1 || H < 1 || W < 1) return TG_ERR_INVALID_ARGUMENT;
    return transpose_entry(src, dst, N, C, (long long)H * W, ival(dtype), stream);
}

tg_status tg_nhwc_to_nchw(const void* src, void* dst, int N, int C, int H, int W,
                          tg_dtype dtype, void* stream) {
    if (N < 1 || C < 1 || H < 1 || W < 1) return TG_ERR_INVALID_ARGUMENT;
    return transpose_entry(src, dst, N, (long long)H * W, C, ival(dtype), stream);
}

tg_status tg_filter_oihw_to_ohwi(const void* src, void* dst, int C_out, int C_in, int kh, int kw,
                                 tg_dtype dtype, void* stream) {
    if (C_out < 1 || C_in < 1 || kh < 1 || kw < 1) return TG_ERR_INVALID_ARGUMENT;
    return transpose_entry(src, dst, C_out, C_in, (long long)kh * kw, ival(dtype), stream);
}

tg_status tg_conv_bn_silu_run(const tg_conv_bn_silu_plan* plan, const void* x, const void* w,
                              const float* bn_scale, const float* bn_bias, void* y,
                              void* workspace, size_t workspace_bytes, void* stream) {
    return run_impl(plan, x, w, bn_scale, bn_bias, nullptr, y, workspace, workspace_bytes, stream);
}

tg_status tg_conv_bn_silu_run_residual(const tg_conv_bn_silu_plan* plan, const void* x,
                                       const void* w, const float* bn_scale, const float* bn_bias,
                                       const void* residual, void* y, void* stream) {
    if (!residual) return TG_ERR_INVALID_ARGUMENT;
    if (plan && (plan->unfused || plan->split || plan->g.out8)) return TG_ERR_UNSUPPORTED;
    return run_impl(plan, x, w, bn_scale, bn_bias, residual, y, nullptr, 0, stream);
}

static bool takes_packed_filter(const tg_conv_bn_silu_plan* plan) {
    return plan->kernel == TG_KERNEL_IGEMM && plan->patch_cfg >= 0 && plan->cu_waves <= 0 &&
           !plan->unfused && !plan->split && plan->dtype == TG_F16 &&
           igemm_patch_packed_bytes(plan->g, plan->patch_cfg) > 0;
}

tg_status tg_conv_bn_silu_packed_filter_bytes(const tg_conv_bn_silu_plan* plan, size_t* bytes) {
    if (!plan || !bytes) return TG_ERR_INVALID_ARGUMENT;
    *bytes = 0;
    if (!takes_packed_filter(plan)) return TG_ERR_UNSUPPORTED;
    *bytes = igemm_patch_packed_bytes(plan->g, plan->patch_cfg);
    return TG_OK;
}

tg_status tg_conv_bn_silu_pack_filter(const tg_conv_bn_silu_plan* plan, const void* w,
                                      void* w_packed, size_t w_packed_bytes, void* stream) {
    if (!plan || !w || !w_packed || w == w_packed) return TG_ERR_INVALID_ARGUMENT;
    if (!takes_packed_filter(plan)) return TG_ERR_UNSUPPORTED;
    if (w_packed_bytes < igemm_patch_packed_bytes(plan->g, plan->patch_cfg))
        return TG_ERR_WORKSPACE;
    if (!aligned16(w) || !aligned16(w_packed)) return TG_ERR_ALIGNMENT;
    hipError_t e = launch_pack_patch_filter(plan->g, plan->patch_cfg, w, w_packed,
                                            (hipStream_t)stream);
    return e == hipSuccess ? TG_OK : TG_ERR_HIP;
}

tg_status tg_conv_bn_silu_run_packed(const tg_conv_bn_silu_plan* plan, const void* x,
                                     const void* w_packed, const float* bn_scale,
                                     const float* bn_bias, void* y, void* stream) {
    if (!plan || !x || !w_packed || !bn_scale || !bn_bias || !y) return TG_ERR_INVALID_ARGUMENT;
    if (!takes_packed_filter(plan)) return TG_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w_packed) || !aligned16(y)) return TG_ERR_ALIGNMENT;
    hipError_t e = launch_igemm_patch(plan->g, plan->patch_cfg, plan->epi, x, w_packed,
                                      bn_scale, bn_bias, y, (hipStream_t)stream, true);
    return e == hipSuccess ? TG_OK : TG_ERR_HIP;
}

tg_status tg_bn_fold(const float* gamma, const float* beta, const float* mean, const float* var,
                     float eps, int C_out, float* bn_scale, float* bn_bias, void* stream) {
    if (!gamma || !beta || !mean || !var || !bn_scale || !bn_bias || C_out < 1 || !(eps >= 0.0f))
        return TG_ERR_INVALID_ARGUMENT;
    hipError_t e = launch_bn_fold(gamma, beta, mean, var, eps, C_out, bn_scale, bn_bias,
                                  (hipStream_t)stream);
    return e == hipSuccess ? TG_OK : TG_ERR_HIP;
}

tg_status tg_conv_bn_silu_query(const tg_conv_bn_silu_plan* plan, int* P, int* Q,
                                tg_kernel* chosen, size_t* workspace_bytes) {
    if (!plan) return TG_ERR_INVALID_ARGUMENT;
    if (P) *P = plan->g.P;
    if (Q) *Q = plan->g.Q;
    if (chosen)
        *chosen = (tg_kernel)(plan->kernel | (plan->unfused ? TG_UNFUSED : 0) |
                              (plan->split ? TG_SPLIT : 0));
    if (workspace_bytes) *workspace_bytes = plan->ws_bytes;
    return TG_OK;
}

tg_status tg_conv_bn_silu_describe(const tg_conv_bn_silu_plan* plan, char* buf, size_t len) {
    if (!plan || !buf) return TG_ERR_INVALID_ARGUMENT;
    if (len == 0) return TG_OK;
    const ConvGeom& g = plan->g;
    char k[160];
    if (plan->kernel == TG_KERNEL_IGEMM && plan->cu_waves > 0) {
        int nb = (g.M + 15) / 16;
        snprintf(k, sizeof(k), "igemm_cu (one workgroup per CU) waves=%d pd=%d grid=%d%s",
                 plan->cu_waves, plan->cu_pd, nb < 256 ? nb : 256, plan->rw_nt ? " nt" : "");
    } else if (plan->kernel == TG_KERNEL_IGEMM && plan->igemm_cfg < 0) {
        snprintf(k, sizeof(k), "igemm_rw (weights in VGPRs) nf=%d cs=%d ncw=%d grid=%d%s",
                 plan->rw_nf, plan->rw_cs, plan->rw_ncw, plan->rw_grid, plan->rw_nt ? " nt" : "");
    } else if (plan->kernel == TG_KERNEL_IGEMM && plan->band) {
        int tpx, tiles, lds;
        igemm_band_describe(g, &tpx, &tiles, &lds);
        snprintf(k, sizeof(k), "igemm_band tile=%dpx x %dch waves=2x2 grid=%d lds=%d",
                 tpx, g.C_out, tiles, lds);
    } else if (plan->kernel == TG_KERNEL_IGEMM && plan->patch_cfg >= 0) {
        int BM, BN, WM, WN, WK;
        int ring;
        igemm_patch_describe(plan->patch_cfg, &BM, &BN, &WM, &WN, &WK, &ring);
        int tiles = g.N * ((g.P * g.Q + BM - 1) / BM) * ((g.C_out + BN - 1) / BN);
        snprintf(k, sizeof(k), "igemm_patch cfg=%d BM=%d BN=%d waves=%dx%dx%d ring=%d grid=%d",
                 plan->patch_cfg, BM, BN, WK, WM, WN, ring, tiles);
    } else if (plan->kernel == TG_KERNEL_IGEMM && plan->dma_cfg >= 0) {
        const IgemmCfg& c = igemm_dma_cfg(plan->dma_cfg);
        int tm = (g.M + c.BM - 1) / c.BM, tn = (g.C_out + c.BN - 1) / c.BN;
        snprintf(k, sizeof(k), "igemm_dma cfg=%d BM=%d BN=%d BK=64 waves=%dx%dx%d grid=%d",
                 plan->dma_cfg, c.BM, c.BN, c.WK, c.WM, c.WN, tm * tn);
    } else if (plan->kernel == TG_KERNEL_IGEMM) {
        const IgemmCfg& c = igemm_cfg(plan->igemm_cfg);
        int tm = (g.M + c.BM - 1) / c.BM, tn = (g.C_out + c.BN - 1) / c.BN;
        snprintf(k, sizeof(k), "igemm cfg=%d BM=%d BN=%d BK=%d waves=%dx%d grid=%d", plan->igemm_cfg,
                 c.BM, c.BN, c.BK, c.WM, c.WN, tm * tn);
    } else if (plan->kernel == TG_KERNEL_TILED && plan->stem_wpc > 0) {
        snprintf(k, sizeof(k), "stem (row bands in LDS, 3 MFMA per 32px x 32ch) wg/CU=%d rows=%d",
                 plan->stem_wpc, plan->stem_rows);
    } else if (plan->kernel == TG_KERNEL_TILED && plan->tm_pipe_grid > 0) {
        snprintf(k, sizeof(k), "tiled_mfma_pipe R=%d grid=%d", plan->tm_rows,
                 plan->tm_pipe_grid);
    } else if (plan->kernel == TG_KERNEL_TILED && plan->tm_rows > 0) {
        int bands = (g.P + plan->tm_rows - 1) / plan->tm_rows;
        snprintf(k, sizeof(k), "tiled_mfma R=%d grid=%d", plan->tm_rows, g.N * bands);
    } else if (plan->kernel == TG_KERNEL_TILED) {
        int bands = (g.P + plan->tiled.R - 1) / plan->tiled.R;
        snprintf(k, sizeof(k), "tiled R=%d lds=%d grid=%d", plan->tiled.R, plan->tiled.lds_bytes,
                 g.N * bands);
    } else {
        snprintf(k, sizeof(k), "scalar grid=%d", (g.M * g.C_out + 255) / 256);
    }
    const char* act = plan->epi == EPI_RELU ? " act=relu"
                      : plan->epi == EPI_GELU ? " act=gelu"
                      : plan->epi == EPI_BN   ? " act=none" : "";
    snprintf(buf, len, "%s%s%s%s %s N=%d H=%d W=%d C_in=%d C_out=%d k=%dx%d s=%d p=%d -> %dx%d",
             plan->unfused ? "unfused:" : (plan->split ? "split:" : ""), k, act,
             plan->g.out8 ? " y=fp8" : "", plan->dtype == TG_F16 ? "f16" : "f32", g.N, g.H,
             g.W, g.C_in, g.C_out, g.kh, g.kw, g.stride, g.pad, g.P, g.Q);
    return TG_OK;
}

tg_status tg_dispatch_choose(int N, int H, int W, int C_in, int C_out, int kh, int kw, int stride,
                             int pad, tg_dtype dtype, tg_dispatch table, tg_kernel* chosen) {
    if (!chosen) return TG_ERR_INVALID_ARGUMENT;
    ConvGeom g;
    tg_status st = make_geom(N, H, W, C_in, C_out, kh, kw, stride, pad, &g);
    if (st != TG_OK) return st;
    const int dt = ival(dtype), tb = ival(table);
    if (dt != TG_F16 && dt != TG_F32) return TG_ERR_UNSUPPORTED;
    if (tb != TG_DISPATCH_MI355X && tb != TG_DISPATCH_PAGES) return TG_ERR_UNSUPPORTED;
    *chosen = dispatch(g, (tg_dtype)dt, (tg_dispatch)tb);
    return TG_OK;
}

const char* tg_status_string(tg_status st) {
    switch (ival(st)) {
        case TG_OK: return "ok";
        case TG_ERR_INVALID_ARGUMENT: return "invalid argument";
        case TG_ERR_UNSUPPORTED: return "unsupported";
        case TG_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
        case TG_ERR_WORKSPACE: return "workspace missing or too small";
        case TG_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* tg_kernel_name(tg_kernel k) {
    int kv = ival(k);
    bool unf = (kv & TG_UNFUSED) != 0, spl = (kv & TG_SPLIT) != 0;
    if (unf && spl) return "unknown kernel";
    switch (kv & ~(TG_UNFUSED | TG_SPLIT)) {
        case TG_KERNEL_AUTO: return unf ? "unfused(auto)" : (spl ? "split(auto)" : "auto");
        case TG_KERNEL_SCALAR:
            return unf ? "unfused(scalar)" : (spl ? "split(scalar)" : "conv2d_bn_silu_scalar");
        case TG_KERNEL_TILED:
            return unf ? "unfused(tiled)" : (spl ? "split(tiled)" : "conv2d_bn_silu_tiled");
        case TG_KERNEL_IGEMM:
            return unf ? "unfused(igemm)" : (spl ? "split(igemm)" : "conv2d_bn_silu_igemm");
    }
    return "unknown kernel";
}

}  // extern "C"
