// C-ABI entry points, configuration table and host dispatch of the gfx950
// fp16 GEMM library.  Declarations and the contract are in include/gemm_f16.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "gemm_f16.h"
#include "pingpong_kernel.h"
#include "skinny_kernel.h"
#include "skinny_splitk_kernel.h"
#include "tile_pipe_kernel.h"

using namespace gk;

namespace {

enum Kind { KIND_TILE = 0, KIND_SKINNY = 1, KIND_SPLITK = 2 };

typedef hipError_t (*launch_fn)(const GemmArgs&, hipStream_t);

struct Config {
    const char* name;
    int kind;
    int bm, bn, bk, wm, wn;  // tile: block tile and wave grid; skinny: bm = 16*MB rows
    int loader;              // tile loaders; -1 for skinny
    int group_m;
    int stages;
    int bslot, dstride, cslot, wpe;  // tile schedule: barrier slot, copy stride, LDS-write slot, waves/SIMD
    int mfma, spread;                // MFMA shape (32: 32x32x16, 16: 16x16x32); schedule flags (skinny: 1 = 16-byte A copies)
    int bt;                          // 1: B given transposed (Bt[N][K])
    int krot;                        // skinny: K stages walked from stage (workgroup mod KT)
    int ksplit;                      // split-K skinny: number of K ranges
    int lds_bytes;
    int threads;
    launch_fn launch[3];     // indexed by epilogue
};

template <int BM, int BN, int BK, int WM, int WN, int ST, int G, int BS, int DS, int LOADER, int CS, int WPE, int MF,
          int SP, int BT, int EPI>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
    dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(WM * WN * 64);
    hipLaunchKernelGGL((gemm_tile_pipe_kernel<BM, BN, BK, WM, WN, ST, G, EPI, BS, DS, LOADER, CS, WPE, MF, SP, BT>),
                       grid, block, 0, s, a);
    return hipGetLastError();
}

template <int MB, int STAGES, int BT, int KROT, int A16, int EPI>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.tiles_n), block(SK_WAVES * 64);
    hipLaunchKernelGGL((gemm_skinny_kernel<MB, STAGES, EPI, BT, KROT, A16>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int G, int BT, int NT, int EPI>
hipError_t launch_pingpong(const GemmArgs& a, hipStream_t s) {
    dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(PP_WAVES * 64);
    hipLaunchKernelGGL((gemm_pingpong_kernel<G, EPI, BT, NT>), grid, block, 0, s, a);
    return hipGetLastError();
}

// Tile config: block tile BM x BN x BK, WM x WN waves, ST LDS stages, tile
// order group G, barrier slot BS, copy stride DS, loader, LDS-write slot CS
// (register loader), waves per SIMD WPE, MFMA shape MF (32 or 16), spread
// LDS reads SP, B transposed BT.
#define TILE_CFG(BM, BN, BK, WM, WN, ST, G, BS, DS, LOADER, CS, WPE, MF, SP, BT, NAME)             \
    Config {                                                                                       \
        NAME, KIND_TILE, BM, BN, BK, WM, WN, LOADER, G, ST, BS, DS, CS, WPE, MF, SP, BT, 0, 0,     \
            TilePipeCfg<BM, BN, BK, WM, WN, ST, MF, BT, ((SP) & 128) ? 1 : 0>::LDS_BYTES, WM * WN * 64, \
        {                                                                                          \
            launch_tile<BM, BN, BK, WM, WN, ST, G, BS, DS, LOADER, CS, WPE, MF, SP, BT, 0>,        \
                launch_tile<BM, BN, BK, WM, WN, ST, G, BS, DS, LOADER, CS, WPE, MF, SP, BT, 1>,    \
                launch_tile<BM, BN, BK, WM, WN, ST, G, BS, DS, LOADER, CS, WPE, MF, SP, BT, 2>     \
        }                                                                                          \
    }

// Ping-pong config (gemm_pingpong_kernel): 256x256 tile, 8 waves in two groups that take turns between the
// 64 MFMAs of a 64-deep stage and the LDS reads and copies of their next one, two stages in LDS, LDS-DMA
// copies; tile order group G, B transposed BT, non-temporal C stores NT.  It reports itself as an LDS-DMA
// tile with BK = 64 and schedule flag 256, and takes whole tiles only (M and N multiples of 256).
#define PINGPONG_CFG(G, BT, NT, NAME)                                                              \
    Config {                                                                                       \
        NAME, KIND_TILE, PP_BM, PP_BN, PP_BK, 2, 4, LOAD_DMA, G, PP_SLOTS, 0, 0, 0, 2, 16,             \
            256 | 32 | ((NT) ? 64 : 0), BT, 0, 0, PP_LDS_BYTES, PP_WAVES * 64,                     \
        {                                                                                          \
            launch_pingpong<G, BT, NT, 0>, launch_pingpong<G, BT, NT, 1>, launch_pingpong<G, BT, NT, 2> \
        }                                                                                          \
    }

// Skinny config: 16*MB rows, ST LDS stages, B transposed BT, rotated K order KR,
// 16-byte A copies A16.
#define SKINNY_CFG(MB, ST, BT, KR, A16, NAME)                                                       \
    Config {                                                                                       \
        NAME, KIND_SKINNY, 16 * MB, SK_BN, SK_BK, 1, SK_WAVES, -1, 1, ST, 0, 0, 0, 1, 16, A16, BT, KR, 0, \
            ST * (16 * MB * SK_BK * 2 + SK_BK * SK_BN * 2), SK_WAVES * 64,                         \
        {                                                                                          \
            launch_skinny<MB, ST, BT, KR, A16, 0>, launch_skinny<MB, ST, BT, KR, A16, 1>,          \
                launch_skinny<MB, ST, BT, KR, A16, 2>                                              \
        }                                                                                          \
    }

template <int MB, int STAGES, int BK, int S, int EPI>
hipError_t launch_splitk(const GemmArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((gemm_skinny_splitk_kernel<MB, STAGES, BK>), dim3((unsigned)(a.tiles_n * a.k_split)),
                       dim3(SKS_WAVES * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t quads = (int64_t)a.M * (a.N / 4);
    hipLaunchKernelGGL((splitk_reduce_kernel<EPI, S>), dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

// Split-K skinny config (B[K][N] only): 16*MB rows, ST LDS stages of BK k-rows, S K ranges.
#define SPLITK_CFG(MB, ST, BK, S, NAME)                                                             \
    Config {                                                                                       \
        NAME, KIND_SPLITK, 16 * MB, SKS_BN, BK, 1, SKS_WAVES, -1, 1, ST, 0, 0, 0, 1, 16, 0, 0, 0, S, \
            ST * (16 * MB * BK * 2 + BK * SKS_BN * 2), SKS_WAVES * 64,                            \
        {                                                                                          \
            launch_splitk<MB, ST, BK, S, 0>, launch_splitk<MB, ST, BK, S, 1>, launch_splitk<MB, ST, BK, S, 2> \
        }                                                                                          \
    }

// The configuration table and the per-shape-class defaults (SEL_*) come from
// a generated include: the offline sweep (sweep.py) writes config_table.inc.
// A different table can be compiled in with -DGEMM_F16_CONFIG_TABLE="file".
#ifndef GEMM_F16_CONFIG_TABLE
#define GEMM_F16_CONFIG_TABLE "config_table.inc"
#endif
#include GEMM_F16_CONFIG_TABLE

const Config kConfigs[] = {GEMM_F16_CONFIGS};
constexpr int kNumConfigs = (int)(sizeof(kConfigs) / sizeof(kConfigs[0]));
static_assert(SEL_SKINNY16 < kNumConfigs && SEL_SKINNY32 < kNumConfigs && SEL_SKINNY64 < kNumConfigs &&
                  SEL_DMA_HUGE < kNumConfigs && SEL_DMA_BIG < kNumConfigs && SEL_DMA_SMALL < kNumConfigs &&
                  SEL_BUF_BIG < kNumConfigs && SEL_BUF_SMALL < kNumConfigs && SEL_REG_BIG < kNumConfigs &&
                  SEL_REG_SMALL < kNumConfigs && SEL_BT_BIG < kNumConfigs && SEL_BT_SMALL < kNumConfigs &&
                  SEL_BT_BUF < kNumConfigs && SEL_BT_REG < kNumConfigs && SEL_BT_SKINNY16 < kNumConfigs &&
                  SEL_BT_SKINNY32 < kNumConfigs && SEL_BT_SKINNY64 < kNumConfigs,
              "shape-class defaults index the table");

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

struct Call {
    int64_t M, N, K;
    const void *A, *B, *bias;
    void* C;
    int epi;
    int64_t lda, ldb, ldc;  // leading dimensions (row strides) in elements
    bool bt = false;        // B given transposed: Bt[N][K], row stride ldb >= K
};

int validate(const Call& c) {
    if (c.M < 0 || c.N < 0 || c.K < 0 || c.M > INT32_MAX || c.N > INT32_MAX || c.K > INT32_MAX)
        return GEMM_ERR_INVALID_DIM;
    if (c.epi < GEMM_EPI_NONE || c.epi > GEMM_EPI_BIAS_GELU) return GEMM_ERR_BAD_EPILOGUE;
    if (c.lda < 0 || c.ldb < 0 || c.ldc < 0 || c.lda > INT32_MAX || c.ldb > INT32_MAX || c.ldc > INT32_MAX)
        return GEMM_ERR_INVALID_DIM;
    if (c.M == 0 || c.N == 0) return GEMM_OK;
    if (c.ldc < c.N || (c.K > 0 && (c.lda < c.K || c.ldb < (c.bt ? c.K : c.N)))) return GEMM_ERR_INVALID_DIM;
    if (!c.C) return GEMM_ERR_NULL_POINTER;
    if (c.K > 0 && (!c.A || !c.B)) return GEMM_ERR_NULL_POINTER;
    if (c.epi != GEMM_EPI_NONE && !c.bias) return GEMM_ERR_NULL_POINTER;
    if (!aligned(c.C, 2) || (c.K > 0 && (!aligned(c.A, 2) || !aligned(c.B, 2))) ||
        (c.epi != GEMM_EPI_NONE && !aligned(c.bias, 2)))
        return GEMM_ERR_MISALIGNED;
    return GEMM_OK;
}

// Whether config `cfg` can run call `c` (validated, M, N > 0).
bool supports(const Config& cfg, const Call& c) {
    if ((cfg.bt != 0) != c.bt) return false;  // each B layout has its own configurations
    const bool epi_bias_ok = (c.epi == GEMM_EPI_NONE) || aligned(c.bias, 8);
    // 16-byte-aligned rows: aligned bases and leading dimensions that are multiples of 8 elements
    const bool vec_ok = aligned(c.A, 16) && aligned(c.B, 16) && aligned(c.C, 16) && c.K % 8 == 0 &&
                        c.N % 8 == 0 && c.lda % 8 == 0 && c.ldb % 8 == 0 && c.ldc % 8 == 0 && epi_bias_ok;
    const int64_t a_end = (c.M - 1) * c.lda + c.K;  // elements from A to the end of its last row
    const int64_t b_end = c.bt ? (c.N - 1) * c.ldb + c.K : (c.K - 1) * c.ldb + c.N;  // same for B (or Bt)
    if (cfg.kind == KIND_SKINNY) {
        // 32-bit buffer offsets: B rows up to K + SK_BK (the last stage's tail), or all of Bt, and all of A
        const bool b_fits = c.bt ? (b_end + SK_BK) * 2 < (int64_t)INT32_MAX
                                 : (c.K + SK_BK) * c.ldb * 2 < (int64_t)INT32_MAX;
        return vec_ok && c.M <= cfg.bm && b_fits && c.M * c.lda * 2 < (int64_t)INT32_MAX;
    }
    if (cfg.kind == KIND_SPLITK) {
        // 32-bit buffer offsets as for the skinny kernel (the last range's stage tail included); the fp32
        // workspace (ranges x M x N) under 2 GiB
        return vec_ok && c.K > 0 && c.M <= cfg.bm && (c.K + cfg.bk) * c.ldb * 2 < (int64_t)INT32_MAX &&
               c.M * c.lda * 2 < (int64_t)INT32_MAX && (int64_t)cfg.ksplit * c.M * c.N * 4 < (int64_t)INT32_MAX;
    }
    if (cfg.loader == LOAD_DMA) {
        // the ping-pong kernel (schedule flag 256) takes whole 256x256 tiles only
        const bool whole = !(cfg.spread & 256) || (c.M % cfg.bm == 0 && c.N % cfg.bn == 0);
        return vec_ok && whole && c.K % cfg.bk == 0 && (int64_t)cfg.bm * c.lda * 2 < (int64_t)INT32_MAX &&
               (int64_t)(c.bt ? cfg.bn : cfg.bk) * c.ldb * 2 < (int64_t)INT32_MAX;
    }
    if (cfg.loader == LOAD_BUF) {
        // 31-bit buffer sizes and offsets: all of A and B, and one stage's tiles.
        const int64_t lim = (int64_t)INT32_MAX - 64;
        const bool fits = c.K > 0 && a_end * 2 < lim && b_end * 2 < lim &&
                          ((int64_t)cfg.bm * c.lda + cfg.bk) * 2 < lim &&
                          (c.bt ? (int64_t)cfg.bn * c.ldb + cfg.bk : (int64_t)cfg.bk * c.ldb + cfg.bn) * 2 < lim;
        // Odd N: B's range is padded by 2 bytes past the end of its last row;
        // allowed only when that end is not on a 4 KiB page boundary, so the
        // pad lies in the page of the last element.
        // (Bt needs no pad: its rows past N are clamped and its k-chunks past K
        // are sent out of range, like A's.)
        const bool pad_ok = c.bt || c.N % 2 == 0 || ((uintptr_t)c.B + (uintptr_t)(b_end * 2)) % 4096 != 0;
        return c.K % 8 == 0 && fits && pad_ok;
    }
    return true;  // register loader: any shape, any 2-byte alignment
}

int pick_default(const Call& c) {
    if (c.bt) {
        if (c.M <= 64) {  // skinny M: bandwidth path streaming Bt once
            const int idx = c.M <= 16 ? SEL_BT_SKINNY16 : (c.M <= 32 ? SEL_BT_SKINNY32 : SEL_BT_SKINNY64);
            if (supports(kConfigs[idx], c)) return idx;
        }
        const int64_t tiles256 = ((c.M + 255) / 256) * ((c.N + 255) / 256);
        const int dma = tiles256 >= 256 ? SEL_BT_BIG : SEL_BT_SMALL;
        if (supports(kConfigs[dma], c)) return dma;
        return supports(kConfigs[SEL_BT_BUF], c) ? SEL_BT_BUF : SEL_BT_REG;
    }
    // skinny M: bandwidth path streaming B once
    if (c.M <= 64) {
        const int idx = c.M <= 16 ? SEL_SKINNY16 : (c.M <= 32 ? SEL_SKINNY32 : SEL_SKINNY64);
        if (supports(kConfigs[idx], c)) return idx;
    }
    const int64_t tiles256 = ((c.M + 255) / 256) * ((c.N + 255) / 256);
    const bool big = tiles256 >= 256;    // at least one 256x256 tile per CU
    const bool huge = tiles256 >= 1024;  // four or more rounds of them
    const int dma = huge ? SEL_DMA_HUGE : (big ? SEL_DMA_BIG : SEL_DMA_SMALL);
    if (supports(kConfigs[dma], c)) return dma;
    // unaligned or ragged: buffer LDS-DMA when K % 8 == 0, else the register loader
    const int buf = big ? SEL_BUF_BIG : SEL_BUF_SMALL;
    if (supports(kConfigs[buf], c)) return buf;
    return big ? SEL_REG_BIG : SEL_REG_SMALL;
}

// Workspace of the split-K path: the fp32 partial sums.  One buffer per device, owned by the library, grown
// (never shrunk) on demand and kept until the process ends.  Work on one stream runs in order, so calls on
// the same stream reuse it freely; a call on another stream first waits, on the device, for the event
// recorded after the previous call's reduce kernel.  The host side of a call holds a mutex, so calls from
// several threads are ordered too.  Growing waits for that event on the host before the old buffer is freed.
struct SplitkWorkspace {
    std::mutex mu;
    void* buf = nullptr;
    size_t cap = 0;
    hipEvent_t done = nullptr;
    hipStream_t last = nullptr;
    bool used = false;
};

SplitkWorkspace& splitk_workspace(int dev) {
    static std::mutex mu;
    static std::vector<SplitkWorkspace*> all;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)all.size() <= dev) all.resize(dev + 1, nullptr);
    if (!all[dev]) all[dev] = new SplitkWorkspace();  // lives until the process ends
    return *all[dev];
}

#if GK_TIMELINE
uint64_t* g_timeline = nullptr;  // stamp buffer of the tile kernels (timeline builds)
#endif

int run(const Config& cfg, const Call& c, hipStream_t stream) {
    GemmArgs a = {};
    a.A = (const f16*)c.A;
    a.B = (const f16*)c.B;
    a.bias = (const f16*)c.bias;
    a.C = (f16*)c.C;
    a.M = (int)c.M;
    a.N = (int)c.N;
    a.K = (int)c.K;
    a.lda = (int)c.lda;
    a.ldb = (int)c.ldb;
    a.ldc = (int)c.ldc;
    if (cfg.kind == KIND_SPLITK) {
        // ranges of whole stages: K rows per range rounded up to the stage depth, and only non-empty ranges
        const int64_t per = (c.K + cfg.ksplit - 1) / cfg.ksplit;
        const int64_t chunk = (per + cfg.bk - 1) / cfg.bk * cfg.bk;
        a.tiles_m = 1;
        a.tiles_n = (int)((c.N + SKS_BN - 1) / SKS_BN);
        a.k_chunk = (int)chunk;
        a.k_split = (int)((c.K + chunk - 1) / chunk);
        const size_t bytes = (size_t)a.k_split * c.M * c.N * sizeof(float);
        int dev = 0;
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return GEMM_ERR_LAUNCH;
        SplitkWorkspace& w = splitk_workspace(dev);
        std::lock_guard<std::mutex> lock(w.mu);
        if (!w.done && hipEventCreateWithFlags(&w.done, hipEventDisableTiming) != hipSuccess) {
            w.done = nullptr;
            return GEMM_ERR_LAUNCH;
        }
        if (w.cap < bytes) {
            if (w.buf) {
                if (w.used && hipEventSynchronize(w.done) != hipSuccess) return GEMM_ERR_LAUNCH;
                (void)hipFree(w.buf);
                w.buf = nullptr;
                w.cap = 0;
            }
            const size_t want = (bytes + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);  // whole MiB
            if (hipMalloc(&w.buf, want) != hipSuccess) {
                w.buf = nullptr;
                return GEMM_ERR_LAUNCH;
            }
            w.cap = want;
        } else if (w.used && w.last != stream && hipStreamWaitEvent(stream, w.done, 0) != hipSuccess) {
            return GEMM_ERR_LAUNCH;
        }
        a.partial = (float*)w.buf;
        const hipError_t e = cfg.launch[c.epi](a, stream);
        if (e != hipSuccess) return GEMM_ERR_LAUNCH;
        if (hipEventRecord(w.done, stream) != hipSuccess) return GEMM_ERR_LAUNCH;
        w.last = stream;
        w.used = true;
        return GEMM_OK;
    }
    if (cfg.kind == KIND_SKINNY) {
        a.tiles_m = 1;
        a.tiles_n = (int)((c.N + SK_BN - 1) / SK_BN);
    } else {
        a.tiles_m = (int)((c.M + cfg.bm - 1) / cfg.bm);
        a.tiles_n = (int)((c.N + cfg.bn - 1) / cfg.bn);
    }
#if GK_TIMELINE
    if (cfg.kind == KIND_TILE && !(cfg.spread & 256)) a.timeline = g_timeline;
#endif
    hipError_t e = cfg.launch[c.epi](a, stream);
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

__global__ void vector_add_f32_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                      float* __restrict__ C, int64_t n) {
    // 16-byte vector body (bases are 16-byte aligned, checked on the host) plus a scalar tail.
    const int64_t n4 = n / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const float4* A4 = (const float4*)A;
    const float4* B4 = (const float4*)B;
    float4* C4 = (float4*)C;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 a = A4[i], b = B4[i];
        C4[i] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    }
    for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) C[i] = A[i] + B[i];
}

__global__ void vector_add_f32_scalar_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                             float* __restrict__ C, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) C[i] = A[i] + B[i];
}

}  // namespace

extern "C" {

#if GK_TIMELINE
// Timeline builds only: the buffer (8 x uint64 per wave, indexed by workgroup and wave) that the tile kernels
// write their clock stamps to; null turns the stamps off.
void gemm_f16_timeline_buffer(void* p) { g_timeline = (uint64_t*)p; }
#endif

const char* gemm_f16_status_string(int status) {
    switch (status) {
        case GEMM_OK: return "GEMM_OK";
        case GEMM_ERR_INVALID_DIM: return "GEMM_ERR_INVALID_DIM";
        case GEMM_ERR_NULL_POINTER: return "GEMM_ERR_NULL_POINTER";
        case GEMM_ERR_BAD_EPILOGUE: return "GEMM_ERR_BAD_EPILOGUE";
        case GEMM_ERR_LAUNCH: return "GEMM_ERR_LAUNCH";
        case GEMM_ERR_NO_CONFIG: return "GEMM_ERR_NO_CONFIG";
        case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED";
        case GEMM_ERR_MISALIGNED: return "GEMM_ERR_MISALIGNED";
        default: return "GEMM_ERR_UNKNOWN";
    }
}

const char* gemm_status_string(int status) { return gemm_f16_status_string(status); }

int gemm_f16_num_configs(void) { return kNumConfigs; }

int gemm_f16_config_info(int idx, char* buf, int buflen) {
    if (idx < 0 || idx >= kNumConfigs) return -GEMM_ERR_NO_CONFIG;
    const Config& c = kConfigs[idx];
    static const char* loaders[] = {"dma", "reg", "buf"};
    char tmp[512];
    int n = snprintf(tmp, sizeof(tmp),
                     "{\"idx\": %d, \"name\": \"%s\", \"kind\": \"%s\", \"bm\": %d, \"bn\": %d, \"bk\": %d, "
                     "\"waves_m\": %d, \"waves_n\": %d, \"loader\": \"%s\", \"group_m\": %d, \"stages\": %d, "
                     "\"bslot\": %d, \"dstride\": %d, \"cslot\": %d, \"waves_per_simd\": %d, "
                     "\"mfma\": %d, \"spread\": %d, \"b_transposed\": %d, \"k_rotate\": %d, \"lds_bytes\": %d, "
                     "\"threads\": %d, \"k_split\": %d}",
                     idx, c.name, c.kind == KIND_TILE ? "tile" : (c.kind == KIND_SKINNY ? "skinny" : "skinny_splitk"),
                     c.bm, c.bn, c.bk, c.wm, c.wn, c.kind == KIND_TILE ? loaders[c.loader] : "lds_dma", c.group_m,
                     c.stages, c.bslot, c.dstride, c.cslot, c.wpe, c.mfma, c.spread, c.bt, c.krot, c.lds_bytes,
                     c.threads, c.ksplit);
    if (buf && buflen > 0) {
        strncpy(buf, tmp, (size_t)buflen - 1);
        buf[buflen - 1] = '\0';
    }
    return n;
}

int gemm_f16_select_config_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                              const void* bias, void* C, int64_t ldc, int epilogue) {
    Call c{M, N, K, A, B, bias, C, epilogue, lda, ldb, ldc};
    int st = validate(c);
    if (st != GEMM_OK) return -st;
    if (M == 0 || N == 0) return -1;
    return pick_default(c);
}

int gemm_f16_select_config(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* bias, void* C,
                           int epilogue) {
    return gemm_f16_select_config_ex(M, N, K, A, K, B, N, bias, C, N, epilogue);
}

int gemm_f16_with_config_ex(int idx, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                            int64_t ldb, const void* bias, void* C, int64_t ldc, int epilogue, void* stream) {
    Call c{M, N, K, A, B, bias, C, epilogue, lda, ldb, ldc};
    int st = validate(c);
    if (st != GEMM_OK) return st;
    if (idx < 0 || idx >= kNumConfigs) return GEMM_ERR_NO_CONFIG;
    if (M == 0 || N == 0) return GEMM_OK;
    if (!supports(kConfigs[idx], c)) return GEMM_ERR_UNSUPPORTED;
    return run(kConfigs[idx], c, (hipStream_t)stream);
}

int gemm_f16_with_config(int idx, int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* bias,
                         void* C, int epilogue, void* stream) {
    return gemm_f16_with_config_ex(idx, M, N, K, A, K, B, N, bias, C, N, epilogue, stream);
}

int gemm_f16_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                const void* bias, void* C, int64_t ldc, int epilogue, void* stream) {
    Call c{M, N, K, A, B, bias, C, epilogue, lda, ldb, ldc};
    int st = validate(c);
    if (st != GEMM_OK) return st;
    if (M == 0 || N == 0) return GEMM_OK;
    return run(kConfigs[pick_default(c)], c, (hipStream_t)stream);
}

int gemm_f16_bt(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* Bt, int64_t ldb,
                const void* bias, void* C, int64_t ldc, int epilogue, void* stream) {
    Call c{M, N, K, A, Bt, bias, C, epilogue, lda, ldb, ldc, true};
    int st = validate(c);
    if (st != GEMM_OK) return st;
    if (M == 0 || N == 0) return GEMM_OK;
    return run(kConfigs[pick_default(c)], c, (hipStream_t)stream);
}

int gemm_f16_bt_select_config(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* Bt, int64_t ldb,
                              const void* bias, void* C, int64_t ldc, int epilogue) {
    Call c{M, N, K, A, Bt, bias, C, epilogue, lda, ldb, ldc, true};
    int st = validate(c);
    if (st != GEMM_OK) return -st;
    if (M == 0 || N == 0) return -1;
    return pick_default(c);
}

int gemm_f16_bt_with_config(int idx, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* Bt,
                            int64_t ldb, const void* bias, void* C, int64_t ldc, int epilogue, void* stream) {
    Call c{M, N, K, A, Bt, bias, C, epilogue, lda, ldb, ldc, true};
    int st = validate(c);
    if (st != GEMM_OK) return st;
    if (idx < 0 || idx >= kNumConfigs) return GEMM_ERR_NO_CONFIG;
    if (M == 0 || N == 0) return GEMM_OK;
    if (!supports(kConfigs[idx], c)) return GEMM_ERR_UNSUPPORTED;
    return run(kConfigs[idx], c, (hipStream_t)stream);
}

int gemm_f16(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* bias, void* C, int epilogue,
             void* stream) {
    return gemm_f16_ex(M, N, K, A, K, B, N, bias, C, N, epilogue, stream);
}

int gemm_f16_time(int idx, int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* bias, void* C,
                  int epilogue, void* stream, int iters, float* median_ms) {
    Call c{M, N, K, A, B, bias, C, epilogue, K, N, N};
    int st = validate(c);
    if (st != GEMM_OK) return st;
    if (!median_ms) return GEMM_ERR_NULL_POINTER;
    if (iters < 1 || iters > GEMM_TIME_MAX_ITERS) return GEMM_ERR_INVALID_DIM;
    if (idx < -1 || idx >= kNumConfigs) return GEMM_ERR_NO_CONFIG;
    if (M == 0 || N == 0) {
        *median_ms = 0.0f;
        return GEMM_OK;
    }
    const int cfg = idx < 0 ? pick_default(c) : idx;
    if (!supports(kConfigs[cfg], c)) return GEMM_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    // iters + 1 events on the stream: event i before launch i, event i + 1 after it
    std::vector<hipEvent_t> ev;
    ev.reserve((size_t)iters + 1);
    st = GEMM_OK;
    for (int i = 0; i <= iters; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) {
            st = GEMM_ERR_LAUNCH;
            break;
        }
        ev.push_back(e);
    }
    if (st == GEMM_OK) st = run(kConfigs[cfg], c, s);  // one untimed launch
    if (st == GEMM_OK && hipEventRecord(ev[0], s) != hipSuccess) st = GEMM_ERR_LAUNCH;
    for (int i = 0; st == GEMM_OK && i < iters; ++i) {
        st = run(kConfigs[cfg], c, s);
        if (st == GEMM_OK && hipEventRecord(ev[i + 1], s) != hipSuccess) st = GEMM_ERR_LAUNCH;
    }
    if (st == GEMM_OK && hipEventSynchronize(ev[iters]) != hipSuccess) st = GEMM_ERR_LAUNCH;
    std::vector<float> t((size_t)iters);
    for (int i = 0; st == GEMM_OK && i < iters; ++i)
        if (hipEventElapsedTime(&t[i], ev[i], ev[i + 1]) != hipSuccess) st = GEMM_ERR_LAUNCH;
    if (st != GEMM_OK && !ev.empty()) hipStreamSynchronize(s);  // no event may be destroyed while pending
    for (hipEvent_t e : ev) hipEventDestroy(e);
    if (st != GEMM_OK) return st;
    std::sort(t.begin(), t.end());
    *median_ms = (iters % 2) ? t[iters / 2] : 0.5f * (t[iters / 2 - 1] + t[iters / 2]);
    return GEMM_OK;
}

int vector_add_f32(int64_t n, const float* A, const float* B, float* C, void* stream) {
    if (n < 0) return GEMM_ERR_INVALID_DIM;
    if (n == 0) return GEMM_OK;
    if (!A || !B || !C) return GEMM_ERR_NULL_POINTER;
    if (!aligned(A, 4) || !aligned(B, 4) || !aligned(C, 4)) return GEMM_ERR_MISALIGNED;
    const int threads = 256;
    const int64_t blocks_needed = (n / 4 + threads - 1) / threads;
    const unsigned blocks = (unsigned)(blocks_needed < 1 ? 1 : (blocks_needed > 256 * 64 ? 256 * 64 : blocks_needed));
    if (aligned(A, 16) && aligned(B, 16) && aligned(C, 16))
        hipLaunchKernelGGL(vector_add_f32_kernel, dim3(blocks), dim3(threads), 0, (hipStream_t)stream, A, B, C, n);
    else
        hipLaunchKernelGGL(vector_add_f32_scalar_kernel, dim3(blocks), dim3(threads), 0, (hipStream_t)stream, A, B, C, n);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // extern "C"
