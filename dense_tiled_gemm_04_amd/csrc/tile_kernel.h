// Tiled fp16 GEMM for gfx950: LDS-staged BM x BK / BK x BN tiles, fp16 MFMA
// (v_mfma_f32_32x32x16_f16) into fp32 accumulators, fused epilogue, one write
// of C.  The structure follows the TileLang tutorial's tiled GEMM (blog post
// "Designing High-Performance GPU Kernels with TileLang", section "Step 4":
// shared tiles A[block_M][block_K] and B[block_K][block_N], a float32
// accumulator fragment, a pipelined K loop) and its fused epilogue (news
// article on TileLang kernel design, paragraph on fusing bias add and GELU
// into the register-resident accumulator), re-designed for CDNA4:
//
//  * workgroup = WM x WN wave64s; each wave owns a (BM/WM) x (BN/WN) sub-tile
//    made of 32x32 MFMA blocks.  The MFMA is issued as D = B^T . A^T (operand
//    a = B fragment, operand b = A fragment) so that each lane's accumulator
//    registers hold 4 consecutive output columns of one row: 8-byte stores.
//  * LDS: two stages of [A tile | B tile], 16-byte chunks XOR-swizzled so
//    that fragment reads hit 64 distinct banks.  A rows are K-contiguous and
//    read with ds_read_b128; B stays row-major [k][n] and is read K-contiguous
//    per lane with the gfx950 transpose read ds_read_b64_tr_b16.
//  * loaders: LOAD_VEC and LOAD_ELEM stage through registers with
//    per-element masking for ragged K / M / N edges and unaligned rows (the
//    aligned fast path with LDS-DMA copies is gemm_tile_dma_kernel).
//  * tile order: XCD-contiguous remap + GROUP_M grouped raster.
#pragma once
#include "common.h"

namespace gk {

enum Loader { LOAD_DMA = 0, LOAD_VEC = 1, LOAD_ELEM = 2 };

template <int BM, int BN, int BK, int WM, int WN, int LOADER, int EPI, int GROUP_M>
struct TileCfg {
    static constexpr int NW = WM * WN;
    static constexpr int NT = NW * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave sub-tile
    static constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA blocks per wave
    static constexpr int CA = BK / 8;                   // 16-byte chunks per A row
    static constexpr int CB = BN / 8;                   // 16-byte chunks per B row
    static constexpr int A_STAGE = BM * BK * 2;         // bytes
    static constexpr int B_STAGE = BK * BN * 2;
    static constexpr int STAGES = 2;
    static constexpr int LDS_BYTES = STAGES * (A_STAGE + B_STAGE);
    static constexpr int RPW_A = 128 / BK;              // A rows per 256-byte bank window
    static_assert(BK % 16 == 0 && BK >= 16 && BK <= 128, "BK");
    static_assert((CA & (CA - 1)) == 0 && (CB & (CB - 1)) == 0, "power-of-two chunk counts");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(CB >= 4, "BN >= 32");
    static_assert((BM * CA) % NT == 0 && (BK * CB) % NT == 0, "tile chunks divisible by threads");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
    static_assert(LOADER == LOAD_VEC || LOADER == LOAD_ELEM, "register-staged loaders only");
};

// A-tile swizzle: logical chunk c of row r lives at chunk c ^ swz_a(r).  Over
// any 16 consecutive rows (one ds_read_b128 quarter-wave), the 16 physical
// positions fall in 16 distinct 16-byte bank groups of the 256-byte window.
template <int BK>
__device__ __forceinline__ int swz_a(int r) {
    constexpr int CA = BK / 8, RPW = 128 / BK;
    return (r / RPW) & (CA - 1);
}
// B-tile swizzle: logical chunk c of k-row kr lives at c ^ swz_b(kr).  A
// transpose read touches 4 consecutive k-rows x 64 bytes per half-wave; XOR
// by 4*(kr mod 4) chunks puts those 16 chunks in distinct bank groups.
template <int BN>
__device__ __forceinline__ int swz_b(int kr) {
    constexpr int CB = BN / 8;
    return (4 * (kr & 3)) & (CB - 1);
}

template <int BM, int BN, int BK, int WM, int WN, int LOADER, int EPI, int GROUP_M>
__global__ void __launch_bounds__(WM* WN * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_tile_kernel(GemmArgs p) {
    using Cfg = TileCfg<BM, BN, BK, WM, WN, LOADER, EPI, GROUP_M>;
    constexpr int NW = Cfg::NW, NT = Cfg::NT, WTM = Cfg::WTM, WTN = Cfg::WTN;
    constexpr int TM = Cfg::TM, TN = Cfg::TN, CA = Cfg::CA, CB = Cfg::CB;
    constexpr int A_STAGE = Cfg::A_STAGE, B_STAGE = Cfg::B_STAGE;

    __shared__ __attribute__((aligned(1024))) char smem_raw[Cfg::LDS_BYTES];
    GK_LDS char* smem = (GK_LDS char*)smem_raw;
    // layout: [A stage 0][A stage 1][B stage 0][B stage 1]
    GK_LDS char* const a_lds = smem;
    GK_LDS char* const b_lds = smem + 2 * A_STAGE;

    const int M = p.M, N = p.N, K = p.K;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int tm, tn;
    {
        const int nwg = p.tiles_m * p.tiles_n;
        const int lid = xcd_contiguous_id((int)blockIdx.x, nwg);
        grouped_tile<GROUP_M>(lid, p.tiles_m, p.tiles_n, tm, tn);
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int KT = (K + BK - 1) / BK;

    // ---------------- fragment read offsets (bytes within a stage) ----------------
    // A operand (MFMA operand b): lane holds A[m = row(lane)][k = 8*(lane/32) .. +7]
    int a_rd[BK / 16];
    {
        const int row = wm * WTM + (lane & 31);
        const int s = swz_a<BK>(row);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            a_rd[kk] = row * BK * 2 + ((c ^ s) << 4);
        }
    }
    // B operand (MFMA operand a) via transpose reads.  Lane L = 16g + 4j + q
    // supplies the address of B[kb + j][nb + 4q .. 4q+3], kb = 8*(g/2) (+16kk,
    // +4h), nb = 16*(g%2) + column base; it receives B[kb + 0..3][nb + (L%16)].
    int b_rd[TN];
    {
        const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
        const int kr = 8 * (g >> 1) + j;
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            const int nl = wn * WTN + ni * 32 + 16 * (g & 1) + 4 * q;
            const int c = nl >> 3;
            b_rd[ni] = kr * BN * 2 + ((c ^ swz_b<BN>(kr)) << 4) + ((nl & 7) << 1);
        }
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TN; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

    // Register fragments of one 16-deep k-step; two sets ping-pong so the
    // LDS reads of step kk+1 are in flight while the MFMAs of step kk run.
    struct Frags {
        f16x8 a[TM];
        f16x8 b[TN];
    };
    auto load_frags = [&](Frags& f, int s, int kk) {
        const GK_LDS char* As = a_lds + s * A_STAGE;
        const GK_LDS char* Bs = b_lds + s * B_STAGE;
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            const GK_LDS char* bp = Bs + b_rd[ni] + 16 * kk * BN * 2;
            f16x4 lo = lds_read_tr16_b64(bp);
            f16x4 hi = lds_read_tr16_b64(bp + 4 * BN * 2);
            f.b[ni] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int mi = 0; mi < TM; ++mi) f.a[mi] = *(const GK_LDS f16x8*)(As + a_rd[kk] + mi * 32 * BK * 2);
    };
    auto mma = [&](const Frags& f) {
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[ni], f.a[mi], acc[mi][ni], 0, 0, 0);
    };
    constexpr int KSTEPS = BK / 16;
    static_assert(KSTEPS % 2 == 0, "k-steps per stage must be even for the fragment ping-pong");

    // Register-staged loads with full masking: any M, N, K; LOAD_VEC also
    // needs 16-byte aligned A/B rows (K % 8 == 0, N % 8 == 0, aligned bases).
    constexpr int A_CH = BM * CA / NT;
    constexpr int B_CH = BK * CB / NT;
    f16x8 ra[A_CH], rb[B_CH];
    auto load_regs = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int t = i * NT + tid;
            const int r = t / CA, c = t % CA;
            const int m = m0 + r, k = k0 + 8 * c;
            const f16* src = p.A + (size_t)m * K + k;
            if (LOADER == LOAD_VEC && m < M && k + 8 <= K) {
                ra[i] = *(const f16x8*)src;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) ra[i][e] = (m < M && k + e < K) ? src[e] : (f16)0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int t = i * NT + tid;
            const int kr = t / CB, c = t % CB;
            const int k = k0 + kr, n = n0 + 8 * c;
            const f16* src = p.B + (size_t)k * N + n;
            if (LOADER == LOAD_VEC && k < K && n + 8 <= N) {
                rb[i] = *(const f16x8*)src;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) rb[i][e] = (k < K && n + e < N) ? src[e] : (f16)0.0f;
            }
        }
    };
    auto store_regs = [&](int s) {
        GK_LDS char* As = a_lds + s * A_STAGE;
        GK_LDS char* Bs = b_lds + s * B_STAGE;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int t = i * NT + tid;
            const int r = t / CA, c = t % CA;
            *(GK_LDS f16x8*)(As + r * BK * 2 + ((c ^ swz_a<BK>(r)) << 4)) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int t = i * NT + tid;
            const int kr = t / CB, c = t % CB;
            *(GK_LDS f16x8*)(Bs + kr * BN * 2 + ((c ^ swz_b<BN>(kr)) << 4)) = rb[i];
        }
    };
    if (KT > 0) {
        load_regs(0);
        store_regs(0);
    }
    Frags f0, f1;
    for (int kt = 0; kt < KT; ++kt) {
        const int s = kt & 1;
        __syncthreads();
        if (kt + 1 < KT) load_regs(kt + 1);
        load_frags(f0, s, 0);
#pragma unroll
        for (int kk = 0; kk + 2 < KSTEPS; kk += 2) {
            load_frags(f1, s, kk + 1);
            mma(f0);
            load_frags(f0, s, kk + 2);
            mma(f1);
        }
        load_frags(f1, s, KSTEPS - 1);
        mma(f0);
        mma(f1);
        if (kt + 1 < KT) store_regs(s ^ 1);
    }

    // ---------------- epilogue: bias / GELU on the accumulators, one write of C ----------------
    // Lane l, register 4*r4 + e of block (mi, ni) holds
    //   C[m0 + wm*WTM + mi*32 + l%32][n0 + wn*WTN + ni*32 + 8*r4 + 4*(l/32) + e].
    constexpr bool VEC_OUT = (LOADER != LOAD_ELEM);  // N % 8 == 0 and C 16-byte aligned
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int n = n0 + wn * WTN + ni * 32 + 8 * r4 + 4 * (lane >> 5);
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (EPI != EPI_NONE) {
                if (VEC_OUT && n + 4 <= N) {
                    f16x4 b4 = *(const f16x4*)(p.bias + n);
#pragma unroll
                    for (int e = 0; e < 4; ++e) bv[e] = (float)b4[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) bv[e] = (n + e < N) ? (float)p.bias[n + e] : 0.f;
                }
            }
#pragma unroll
            for (int mi = 0; mi < TM; ++mi) {
                const int m = m0 + wm * WTM + mi * 32 + (lane & 31);
                if (m >= M) continue;
                f16x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = (f16)apply_epilogue<EPI>(acc[mi][ni][4 * r4 + e], bv[e]);
                f16* dst = p.C + (size_t)m * N + n;
                if (VEC_OUT && n + 4 <= N) {
                    *(f16x4*)dst = o;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) dst[e] = o[e];
                }
            }
        }
    }
}

}  // namespace gk
