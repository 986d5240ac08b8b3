// Pipelined tile kernel of the fp16 GEMM on gfx950.
//
// It computes the tutorial's tiled GEMM: fp16 tiles A[block_M][block_K] and
// B[block_K][block_N] staged in shared memory, a float32 register accumulator,
// a pipelined K loop and the fused bias/GELU epilogue. The sources are the
// blog post "Designing High-Performance GPU Kernels with TileLang", section
// "Step 4", and the news article on TileLang kernel design, paragraphs on the
// tiled GEMM and on the fused epilogue.
//
// What is specific to CDNA4:
//  * MFMA. v_mfma_f32_32x32x16_f16 (MF = 32) or v_mfma_f32_16x16x32_f16
//    (MF = 16). The 16x16 form moves about a fifth less register data per
//    FLOP (a quarter of the accumulator per MFMA), which lets the chip hold a
//    higher clock under its power limit. Either is issued as
//    C^T = B^T . A^T, so each lane holds 4 consecutive columns of one output
//    row. A fragments come from ds_read_b128. B fragments come from row-major
//    [k][n] LDS by the transpose read ds_read_b64_tr_b16. Both tiles are
//    XOR-swizzled in 16-byte chunks so that the reads are free of bank
//    conflicts.
//  * Schedule. Every MFMA slot is fenced with sched_barrier, so the issue
//    order is exactly the one written here:
//      slot i of a k-step: MFMA i, the LDS reads scheduled for slot i (the
//      next k-step's fragments, either one per slot from slot 0 or, with
//      SPREAD, spread evenly over the k-step), and the copy work scheduled
//      for slot i.
//    At slot BSLOT of a stage's last k-step, the wave waits for its part of
//    stage kt+1, and one barrier publishes it. All LDS reads of stage kt have
//    landed by then, so the same barrier also frees stage kt's buffer. The
//    next stage's first fragments are then read in the remaining slots.
//  * Copies, two loaders:
//    - LOAD_DMA: HBM/L2 -> LDS by LDS-DMA (global_load_lds_dwordx4), so no
//      VGPR is spent on staging. STAGES ring buffers. The copies of stage
//      kt+STAGES-1 are issued at every DSTRIDE-th slot of stage kt.
//      Requires K % BK == 0, N % 8 == 0, 16-byte-aligned rows of A, B and C
//      (bases and leading dimensions) and an 8-byte-aligned bias. Rows past M re-read row M-1, and columns past N
//      re-read the last chunk; neither is stored.
//    - LOAD_BUF: the same LDS-DMA ring, issued through buffer resources
//      (buffer_load_dwordx4 ... lds), for unaligned shapes: any M and N,
//      K % 8 == 0, any 2-byte alignment of A, B, C and bias. The hardware
//      range check of a buffer load works per dword: a dword whose last byte
//      lies at or past num_records reads as zero. B's resource ends at the
//      end of B, so the k-rows past K of the last stage read as zeros. Its
//      num_records is padded by 2 bytes when N is odd, because there a chunk
//      that holds the last element of B can start 2 bytes off the dword grid
//      of the end. The host only allows that pad when it stays inside the
//      page of the last element. Columns past N read the next row; they
//      reach only output columns past N, which are never stored. A chunks at
//      k >= K are redirected to an offset past num_records and read as zeros
//      (K % 8 == 0, so no chunk straddles K). Rows past M re-read row M-1.
//    - LOAD_REG: any M, N, K and any 2-byte alignment. Two LDS stages and one
//      set of staging registers. In stage kt, slot CSLOT+j writes register j
//      (stage kt+1, loaded one stage earlier) to LDS with ds_write_b128, and
//      slot CSLOT+j*DSTRIDE then reloads it with stage kt+2. So every load
//      has about a stage to land. The loads are 16-byte loads; the hardware
//      accepts unaligned addresses. Element-wise loads are used only for a
//      chunk that straddles the end of a row (N) or of K. Zeros are written
//      past K (in both A and B) and past N, and rows past M are clamped.
//  * BT = 1: B is given transposed, Bt[N][K] row-major (the layout of a linear
//    layer's weight), and C = A . Bt^T.  Its tiles [BN][BK] are copied, laid
//    out and read exactly like A's (K-contiguous rows, ds_read_b128), with rows
//    past N clamped and (LOAD_BUF) k-chunks past K sent out of range.
//  * Tile order. XCD-contiguous remap of the workgroup id, then a grouped
//    raster of GROUP_M tile-rows (GROUP_M = 1: row-major after the remap;
//    GROUP_M = 0: row-major without the remap, the unswizzled baseline).
//  * Epilogue. Bias and GELU run in fp32 on the accumulators; with the LDS
//    epilogue (SPREAD bit 5) the fp16 tile is then staged in the freed stage
//    buffers and written back as row-contiguous 16-byte stores (optionally
//    non-temporal, bit 6), since in a one-round grid every workgroup reaches
//    its epilogue at once and the C write is exposed in full.
#pragma once
#include "common.h"

namespace gk {

enum Loader { LOAD_DMA = 0, LOAD_REG = 1, LOAD_BUF = 2 };

// A-tile swizzle: logical chunk c of row r lives at chunk c ^ swz_a(r).  Over
// any 16 consecutive rows (one ds_read_b128 quarter-wave), the 16 physical
// positions fall in 16 distinct 16-byte bank groups of the 256-byte window.
template <int BK>
__device__ __forceinline__ int swz_a(int r) {
    constexpr int CA = BK / 8, RPW = 128 / BK;
    return (r / RPW) & (CA - 1);
}
// B-tile swizzle: logical chunk c of k-row kr lives at c ^ swz_b(kr).
//  MF = 32: a transpose read touches 4 consecutive k-rows x 64 bytes per
//  half-wave; XOR by 4*(kr mod 4) chunks puts those 16 chunks in distinct
//  bank groups.
//  MF = 16: a half-wave touches rows {8g + 4h + j : j < 4} for two
//  consecutive g, two chunks per row; XOR by an even value made of (kr mod 4)
//  and bit 3 of kr spreads those 16 chunks over distinct bank groups.
//  Row widths that are a multiple of 8 chunks but not a power of two (BN =
//  192: 384-byte rows, so consecutive rows start half a 256-byte bank window
//  apart) use XOR values below 8, which keep a chunk inside its aligned group
//  of 8 and so inside the row. Rows r and r+1 are already half a window apart,
//  so only pairs of rows need separating: XOR by 4 for MF = 32, and for MF = 16
//  by 2 * ((r/2) mod 2) + 4 * ((r/8) mod 2).
template <int BN, int MF>
__device__ __forceinline__ int swz_b(int kr) {
    constexpr int CB = BN / 8;
    if constexpr ((CB & (CB - 1)) != 0) {
        static_assert(CB % 8 == 0 && (BN * 2) % 256 == 128, "non-power-of-two rows: 128-byte offset per row");
        if constexpr (MF == 32) {
            return 4 * ((kr >> 1) & 1);
        } else {
            return 2 * ((kr >> 1) & 1) + 4 * ((kr >> 3) & 1);
        }
    } else if constexpr (MF == 32) {
        return (4 * (kr & 3)) & (CB - 1);
    } else {
        return (2 * ((kr & 3) | (((kr >> 3) & 1) << 2))) & (CB - 1);
    }
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int MF = 32, int BT = 0, int AXS = 0>
struct TilePipeCfg {
    static constexpr int NW = WM * WN;
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave sub-tile
    static constexpr int TM = WTM / MF, TN = WTN / MF;  // MFxMF MFMA blocks per wave
    static constexpr int KS = MF == 32 ? 16 : 32;       // k per MFMA
    static constexpr int CA = BK / 8, CB = BN / 8;      // 16-byte chunks per A / B row
    static constexpr int A_STAGE = BM * BK * 2, B_STAGE = BK * BN * 2;
    static constexpr int LDS_BYTES = (STAGES + AXS) * A_STAGE + STAGES * B_STAGE;  // AXS: extra A stages
    static constexpr int KSTEPS = BK / KS;              // k-steps per stage
    static constexpr int A_INS = BM * CA / 64 / NW;     // 16-byte copies per lane and stage
    static constexpr int B_INS = BT ? BN * CA / 64 / NW : BK * CB / 64 / NW;
    static constexpr int PER_STAGE = A_INS + B_INS;
    static constexpr int NMMA = TM * TN;                // MFMAs (slots) per k-step
    static constexpr int NB = BT ? TN : 2 * TN;         // B fragment reads per k-step
    static constexpr int NRD = TM + NB;                 // LDS reads per k-step
    static_assert(MF == 32 || MF == 16, "MFMA shape");
    static_assert(KSTEPS % 2 == 0, "even k-steps per stage (fragment ping-pong)");
    static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile of whole MFMA blocks");
    static_assert((CA & (CA - 1)) == 0 && CB >= 4 && ((CB & (CB - 1)) == 0 || CB % 8 == 0), "chunk counts");
    static_assert((BM * CA) % (64 * NW) == 0 && (BT ? BN * CA : BK * CB) % (64 * NW) == 0, "copy split over waves");
    static_assert(STAGES >= 2 && PER_STAGE * (STAGES - 1) <= 63, "vmcnt range");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
};

// Slot of LDS read j (0 <= j < NRD) among `avail` slots starting at `first`:
// one per slot while they fit (unless SPREAD), otherwise spread evenly.
template <int NRD, int SPREAD>
__device__ constexpr int read_slot(int j, int first, int avail) {
    return first + (NRD <= avail && !SPREAD ? j : j * avail / NRD);
}

typedef f16x8 f16x8_u __attribute__((aligned(2)));
typedef f16x4 f16x4_u __attribute__((aligned(2)));

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int GROUP_M, int EPI, int BSLOT, int DSTRIDE,
          int LOADER, int CSLOT, int WPE, int MF, int SPREAD, int BT>
__global__ void __launch_bounds__(WM* WN * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
gemm_tile_pipe_kernel(GemmArgs p) {
    uint64_t tl[8] = {};  // timeline builds: shader clock at the 4 points, then the real-time counter
    auto stamp = [&](int k) {
        if constexpr (GK_TIMELINE) {
            tl[k] = __builtin_amdgcn_s_memtime();
            tl[4 + k] = __builtin_amdgcn_s_memrealtime();
        }
    };
    stamp(0);
    using Cfg = TilePipeCfg<BM, BN, BK, WM, WN, STAGES, MF, BT, (SPREAD & 128) ? 1 : 0>;
    constexpr int KS = Cfg::KS;
    constexpr int NW = Cfg::NW, WTM = Cfg::WTM, WTN = Cfg::WTN, TM = Cfg::TM, TN = Cfg::TN;
    constexpr int CA = Cfg::CA, CB = Cfg::CB, A_STAGE = Cfg::A_STAGE, B_STAGE = Cfg::B_STAGE;
    constexpr int KSTEPS = Cfg::KSTEPS, A_INS = Cfg::A_INS, B_INS = Cfg::B_INS, PER_STAGE = Cfg::PER_STAGE;
    constexpr int NMMA = Cfg::NMMA, NRD = Cfg::NRD, NB = Cfg::NB;
    constexpr int LAST = (KSTEPS - 1) * NMMA + BSLOT;  // stage slot of the barrier
    constexpr bool RING = LOADER != LOAD_REG;          // LDS-DMA ring of STAGES buffers
    static_assert(BSLOT >= 0 && BSLOT + 1 < NMMA, "barrier slot inside the last k-step, reads after it");
    // EARLY (SPREAD bit 3): the copies of stage kt+STAGES go into stage kt's own
    // buffer right after stage kt's barrier (every wave's reads of it have
    // completed there), instead of the copies of stage kt+STAGES-1 being
    // issued from slot 0 of stage kt.  Each copy then has the rest of stage
    // kt plus stage kt+1 up to its barrier to land.
    constexpr bool EARLY = (SPREAD & 8) != 0;
    static_assert(EARLY || (DSTRIDE >= 1 && (PER_STAGE - 1) * DSTRIDE < LAST), "every copy is issued before the barrier");
    static_assert(!EARLY || (RING && DSTRIDE >= 1 && LAST + 1 + (PER_STAGE - 1) * DSTRIDE < KSTEPS * NMMA),
                  "early copies: ring loaders, all issued after the barrier within the stage");
    static_assert(RING || (STAGES == 2 && CSLOT >= 0 && CSLOT + PER_STAGE <= LAST + 1 &&
                                         CSLOT + (PER_STAGE - 1) * DSTRIDE < KSTEPS * NMMA),
                  "register loader: 2 stages; every LDS write precedes the barrier; every reload fits "
                  "in the stage");

    __shared__ __attribute__((aligned(1024))) char smem_raw[Cfg::LDS_BYTES];
    GK_LDS char* const a_lds = (GK_LDS char*)smem_raw;           // [STAGES][BM][BK]
    // AX (SPREAD bit 7): the A ring is one stage deeper than the B ring.
    constexpr bool AX = (SPREAD & 128) != 0;
    constexpr int SA = STAGES + (AX ? 1 : 0);                    // A ring depth
    GK_LDS char* const b_lds = a_lds + SA * A_STAGE;             // [STAGES][BK][BN]

    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb, ldc = p.ldc;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    if constexpr (GROUP_M == 0) {
        // plain row-major tile order, no XCD remap (the unswizzled baseline of the tile-order ablation)
        tm = (int)blockIdx.x / p.tiles_n;
        tn = (int)blockIdx.x % p.tiles_n;
    } else {
        const int nwg = p.tiles_m * p.tiles_n;
        grouped_tile<GROUP_M>(xcd_contiguous_id((int)blockIdx.x, nwg), p.tiles_m, p.tiles_n, tm, tn);
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int KT = (K + BK - 1) / BK;

    // Fragment read offsets (bytes within a stage).
    // A (MFMA operand b): lane holds A[m = row(lane)][k = KS kk + 8 (lane / MF) .. +7],
    // row(lane) = lane % MF within the block.
    int a_rd[KSTEPS];
    {
        const int row = wm * WTM + (lane % MF);
        const int s = swz_a<BK>(row);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            a_rd[kk] = row * BK * 2 + ((((KS / 8) * kk + lane / MF) ^ s) << 4);
    }
    // B (MFMA operand a) by transpose reads: lane L = 16g + 4j + q gives the
    // address of B[kb + j][nb + 4q .. 4q+3] and receives B[kb + 0..3][nb + L%16].
    // MF = 32: kb = 8 (g / 2) (+ 16 kk + 4 h), nb = 16 (g % 2) within a 32-column block;
    // MF = 16: kb = 8 g (+ 32 kk + 4 h), nb = 0 within a 16-column block.
    // Neither the k-step nor the half h changes the swizzle of the row.
    int b_rd[BT ? 1 : TN];
    if constexpr (!BT) {
        const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
        const int kr = (MF == 32 ? 8 * (g >> 1) : 8 * g) + j;
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            const int nl = wn * WTN + ni * MF + (MF == 32 ? 16 * (g & 1) : 0) + 4 * q;
            b_rd[ni] = kr * BN * 2 + (((nl >> 3) ^ swz_b<BN, MF>(kr)) << 4) + ((nl & 7) << 1);
        }
    }
    // BT: B is held transposed, Bt[n][k], and its LDS tile [BN][BK] is laid out
    // and read exactly like A's: lane l reads Bt[n = row(l)][KS kk + 8 (l / MF) .. +7].
    int bt_rd[BT ? KSTEPS : 1];
    if constexpr (BT) {
        const int row = wn * WTN + (lane % MF);
        const int s = swz_a<BK>(row);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            bt_rd[kk] = row * BK * 2 + ((((KS / 8) * kk + lane / MF) ^ s) << 4);
    }

    // Copy j (0 <= j < PER_STAGE) of a stage: destination chunk
    // P = (i * NW + wave) * 64 + lane of the A (j < A_INS, i = j) or the B
    // (i = j - A_INS) tile, which is lane-contiguous; its source is the
    // logical chunk that the swizzle puts at P.
    // Copy sources.  LOAD_DMA: byte offsets from the tile origin of the stage
    // (rows clamped to M-1, columns to the last chunk).  LOAD_BUF: the same
    // with unclamped columns, plus the k offset of each A chunk.  LOAD_REG:
    // per chunk, the k offset in the stage and the row pointer (rows clamped
    // to M-1) for A, the k-row and column for B.
    uint32_t a_off[A_INS], b_off[B_INS];
    int a_ck[A_INS], b_kr[B_INS], b_cn[B_INS], b_ck[B_INS];
    const f16* a_row[A_INS];
    const f16* b_row[B_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int P = (i * NW + wave) * 64 + lane;
        const int r = P / CA, c = (P % CA) ^ swz_a<BK>(r);
        const int m = min(m0 + r, M - 1);
        if constexpr (RING) a_off[i] = (uint32_t)(((m - m0) * lda + 8 * c) * 2);
        if constexpr (LOADER != LOAD_DMA) a_ck[i] = 8 * c;
        if constexpr (LOADER == LOAD_REG) {
            a_row[i] = p.A + (size_t)m * lda;
        }
    }
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        const int P = (i * NW + wave) * 64 + lane;
        if constexpr (BT) {  // as for A: row n of Bt (clamped to N-1), k chunk c
            const int r = P / CA, c = (P % CA) ^ swz_a<BK>(r);
            const int n = min(n0 + r, N - 1);
            if constexpr (RING) b_off[i] = (uint32_t)(((n - n0) * ldb + 8 * c) * 2);
            if constexpr (LOADER != LOAD_DMA) b_ck[i] = 8 * c;
            if constexpr (LOADER == LOAD_REG) b_row[i] = p.B + (size_t)n * ldb;
        } else {
            const int kr = P / CB, c = (P % CB) ^ swz_b<BN, MF>(kr);
            if constexpr (LOADER == LOAD_DMA) {
                const int n = min(n0 + 8 * c, N - 8) - n0;
                b_off[i] = (uint32_t)((kr * ldb + n) * 2);
            } else if constexpr (LOADER == LOAD_BUF) {
                b_off[i] = (uint32_t)((kr * ldb + 8 * c) * 2);
            } else {
                b_kr[i] = kr;
                b_cn[i] = n0 + 8 * c;
            }
        }
    }
    const char* const a_row0 = (const char*)(p.A + (size_t)m0 * lda);
    // origin of the B tile: column n0 of B, or row n0 of Bt
    const char* const b_col0 = (const char*)(BT ? p.B + (size_t)n0 * ldb : p.B + n0);
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t a_lds0 = lds_addr(a_lds) + wave_s * 64 * 16;
    const uint32_t b_lds0 = lds_addr(b_lds) + wave_s * 64 * 16;

    // LOAD_BUF: buffer resources of stage kt.  A: from the stage's tile origin
    // to the end of A's last row.  B: from the stage's tile origin to the end
    // of B's last row (plus the 2-byte pad for odd N).  Both byte counts fit
    // 31 bits (host check).
    const int b_pad = (N & 1) ? 2 : 0;
    auto rsrc_a = [&](int kt) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(a_row0 + (size_t)kt * BK * 2), (short)0,
                                                 ((M - 1 - m0) * lda + K) * 2 - kt * BK * 2, 0x00020000);
    };
    auto rsrc_b = [&](int kt) {
        if constexpr (BT) {  // to the end of Bt's last row, like A
            return __builtin_amdgcn_make_buffer_rsrc((void*)(b_col0 + (size_t)kt * BK * 2), (short)0,
                                                     ((N - 1 - n0) * ldb + K) * 2 - kt * BK * 2, 0x00020000);
        } else {
            return __builtin_amdgcn_make_buffer_rsrc((void*)(b_col0 + (size_t)kt * BK * ldb * 2), (short)0,
                                                     ((K - 1) * ldb + N) * 2 + b_pad - n0 * 2 - kt * BK * ldb * 2,
                                                     0x00020000);
        }
    };
    // Ring loaders: copy j of stage kt into ring buffer sa (an A copy, j < A_INS) or sb (a B copy).
    auto dma_op = [&](int j, int kt, int sa, int sb) {
        if (j < A_INS) {
            const uint32_t lds = a_lds0 + sa * A_STAGE + j * NW * 64 * 16;
            if constexpr (LOADER == LOAD_BUF) {
                dma_buffer_16(rsrc_a(kt), a_ck[j] < K - kt * BK ? a_off[j] : 0x80000000u, lds);
            } else {
                dma_global_16(a_row0 + (size_t)kt * BK * 2, a_off[j], lds);
            }
        } else {
            const int i = j - A_INS;
            const uint32_t lds = b_lds0 + sb * B_STAGE + i * NW * 64 * 16;
            if constexpr (LOADER == LOAD_BUF && BT) {
                dma_buffer_16(rsrc_b(kt), b_ck[i] < K - kt * BK ? b_off[i] : 0x80000000u, lds);
            } else if constexpr (LOADER == LOAD_BUF) {
                dma_buffer_16(rsrc_b(kt), b_off[i], lds);
            } else if constexpr (BT) {
                dma_global_16(b_col0 + (size_t)kt * BK * 2, b_off[i], lds);
            } else {
                dma_global_16(b_col0 + (size_t)kt * BK * ldb * 2, b_off[i], lds);
            }
        }
    };
    // LOAD_REG: load copy j of stage kt into a register, then write it to LDS.
    f16x8 stg[LOADER == LOAD_REG ? PER_STAGE : 1];
    auto gload_op = [&](int j, int kt) {
        f16x8 v = {};
        if (j < A_INS) {
            const int k = kt * BK + a_ck[j];
            const f16* src = a_row[j] + k;
            if (k + 8 <= K) {
                v = *(const f16x8_u*)src;
            } else if (k < K) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (k + e < K) v[e] = src[e];
            }
        } else if constexpr (BT) {
            const int i = j - A_INS;
            const int k = kt * BK + b_ck[i];
            const f16* src = b_row[i] + k;
            if (k + 8 <= K) {
                v = *(const f16x8_u*)src;
            } else if (k < K) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (k + e < K) v[e] = src[e];
            }
        } else {
            const int i = j - A_INS;
            const int k = kt * BK + b_kr[i], n = b_cn[i];
            const f16* src = p.B + (size_t)k * ldb + n;
            if (k < K) {
                if (n + 8 <= N) {
                    v = *(const f16x8_u*)src;
                } else if (n < N) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < N) v[e] = src[e];
                }
            }
        }
        stg[LOADER == LOAD_REG ? j : 0] = v;
    };
    auto lwrite_op = [&](int j, int sb) {
        GK_LDS char* dst = (j < A_INS) ? a_lds + sb * A_STAGE + ((j * NW + wave) * 64 + lane) * 16
                                       : b_lds + sb * B_STAGE + (((j - A_INS) * NW + wave) * 64 + lane) * 16;
        *(GK_LDS f16x8*)dst = stg[LOADER == LOAD_REG ? j : 0];
    };

    constexpr int NACC = MF * MF / 64;  // fp32 accumulators per lane and block
    typedef float accv __attribute__((ext_vector_type(NACC)));
    accv acc[TM][TN];
#pragma unroll
    for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TN; ++ni)
#pragma unroll
            for (int r = 0; r < NACC; ++r) acc[mi][ni][r] = 0.0f;

    // Two fragment sets: the reads of k-step kk+1 land in one while the MFMAs
    // of k-step kk consume the other.  Read j: 0 -> A[0]; 1..NB -> B (halves of
    // B[(j-1)/2] by transpose reads, or Bt[j-1] whole with BT); then A[1..TM-1]
    // -- the order in which MFMA row 0 needs them.
    // INPLACE (SPREAD bit 1): B keeps two sets, A only one.  MFMA slot i uses
    // A[i / TN], so A[mi] is free after slot (mi+1) TN - 1 and is refilled
    // there with the next k-step's row mi; A[TM-1], busy to the end of the
    // k-step, is refilled at slot 0 of the k-step that needs it, (TM-1) TN
    // slots ahead of its first use.  That saves TM fragment registers, which
    // keeps the 16x16 schedules' accumulators in place.
    constexpr bool INPLACE = (SPREAD & 2) != 0;
    constexpr bool PINNED = (SPREAD & 4) != 0;
    // FRONTB (SPREAD bit 4, with INPLACE): the next k-step's B reads go in the
    // first slots of the k-step (after the barrier on a stage's last k-step)
    // rather than spread over it, since the next k-step's first MFMA row needs
    // every B fragment within its first TN slots.
    constexpr int BSPREAD = (SPREAD & 16) ? 0 : 1;
    static_assert(!(SPREAD & 16) || INPLACE, "front-loaded B reads belong to the in-place schedule");
    static_assert(!AX || (RING && EARLY && INPLACE && STAGES == 2), "deeper A ring: ring loaders, early copies, "
                  "in-place A, two B stages");
    static_assert(!INPLACE || TM >= 2, "in-place A refill needs two MFMA rows");
    f16x8 fa[INPLACE ? 1 : 2][TM];
    f16x4 fb[2][BT ? 1 : TN][2];
    f16x8 fbt[2][BT ? TN : 1];
    auto read_op = [&](int set, int j, int sb, int kk) {
        const GK_LDS char* As = a_lds + sb * A_STAGE;
        const GK_LDS char* Bs = b_lds + sb * B_STAGE;
        if (j == 0) {
            fa[set][0] = *(const GK_LDS f16x8*)(As + a_rd[kk]);
        } else if (j <= NB) {
            if constexpr (BT) {
                const int ni = j - 1;
                fbt[set][ni] = *(const GK_LDS f16x8*)(Bs + bt_rd[kk] + ni * MF * BK * 2);
            } else {
                const int ni = (j - 1) / 2, h = (j - 1) % 2;
                fb[set][ni][h] = lds_read_tr16_b64(Bs + b_rd[ni] + (KS * kk + 4 * h) * BN * 2);
            }
        } else {
            const int mi = j - NB;
            fa[set][mi] = *(const GK_LDS f16x8*)(As + a_rd[kk] + mi * MF * BK * 2);
        }
    };
    // INPLACE reads: A row mi into the single A set, B read jb (0 <= jb < NB) into set `set`.
    auto read_a = [&](int mi, int sb, int kk) {
        fa[0][mi] = *(const GK_LDS f16x8*)(a_lds + sb * A_STAGE + a_rd[kk] + mi * MF * BK * 2);
    };
    auto read_b = [&](int set, int jb, int sb, int kk) {
        const GK_LDS char* Bs = b_lds + sb * B_STAGE;
        if constexpr (BT) {
            fbt[set][jb] = *(const GK_LDS f16x8*)(Bs + bt_rd[kk] + jb * MF * BK * 2);
        } else {
            fb[set][jb / 2][jb % 2] = lds_read_tr16_b64(Bs + b_rd[jb / 2] + (KS * kk + 4 * (jb % 2)) * BN * 2);
        }
    };
    auto mma_op = [&](int set, int i) {
        const int mi = i / TN, ni = i % TN;
        const int aset = INPLACE ? 0 : set;
        f16x8 b;
        if constexpr (BT) {
            b = fbt[set][ni];
        } else {
            b = __builtin_shufflevector(fb[set][ni][0], fb[set][ni][1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
        if constexpr (PINNED && MF == 32) {
            asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc[mi][ni]) : "v"(b), "v"(fa[aset][mi]));
        } else if constexpr (PINNED) {
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc[mi][ni]) : "v"(b), "v"(fa[aset][mi]));
        } else if constexpr (MF == 32) {
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, fa[aset][mi], acc[mi][ni], 0, 0, 0);
        } else {
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, fa[aset][mi], acc[mi][ni], 0, 0, 0);
        }
    };

    // Prologue: stages 0 .. STAGES-2 (EARLY: 0 .. STAGES-1) in LDS or in
    // flight, then stage 0's first fragments.
    if constexpr (RING) {
        constexpr int PRE = EARLY ? STAGES : STAGES - 1;
#pragma unroll
        for (int st = 0; st < PRE; ++st)
            if (st < KT)
#pragma unroll
                for (int j = 0; j < PER_STAGE; ++j) dma_op(j, st, st, st);
        if constexpr (AX) {  // A of stage 2 as well; stage 0 has landed when A1, B1 and A2 may remain
            if (KT > 2) {
#pragma unroll
                for (int j = 0; j < A_INS; ++j) dma_op(j, 2, 2, 0);
                wait_vmcnt<PER_STAGE + A_INS>();
            } else {
                wait_vmcnt0();
            }
        } else if (KT >= PRE) {
            wait_vmcnt<(PRE - 1) * PER_STAGE>();
        } else {
            wait_vmcnt0();
        }
    } else {
        if (KT > 0) {
#pragma unroll
            for (int j = 0; j < PER_STAGE; ++j) gload_op(j, 0);
#pragma unroll
            for (int j = 0; j < PER_STAGE; ++j) lwrite_op(j, 0);
        }
        if (KT > 1) {
#pragma unroll
            for (int j = 0; j < PER_STAGE; ++j) gload_op(j, 1);
        }
    }
    __syncthreads();
    stamp(1);
    if constexpr (GK_TIMELINE) {  // the first two stamps go out now, so none stays live across the K loop
        if (p.timeline != nullptr && (threadIdx.x & 63) == 0) {
            uint64_t* o = p.timeline + ((size_t)blockIdx.x * (WM * WN) + (threadIdx.x >> 6)) * 8;
            o[0] = tl[0];
            o[1] = tl[1];
            o[4] = tl[4];
            o[5] = tl[5];
        }
    }
    if (KT > 0) {
        if constexpr (INPLACE) {  // A[TM-1] is read at slot 0 of the k-step
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) read_b(0, jb, 0, 0);
#pragma unroll
            for (int mi = 0; mi + 1 < TM; ++mi) read_a(mi, 0, 0);
        } else {
#pragma unroll
            for (int j = 0; j < NRD; ++j) read_op(0, j, 0, 0);
        }
    }

    int s = 0;   // ring buffer of the stage being computed (B; A too unless AX)
    int sa = 0;  // AX: A ring buffer of the stage being computed
    // PHASE 2: every stage the copies of this stage refer to exists (ring
    // loaders: kt+STAGES-1, or kt+STAGES with EARLY; LOAD_REG: kt+1 written
    // and kt+2 loaded), so they
    // are issued unconditionally and the DMA wait count is exact.  PHASE 1
    // (LOAD_REG only): the last write, no reload.  PHASE 0: no copy work; the
    // ring loaders wait for everything.
    auto stage = [&]<int PHASE>(int kt) {
        const bool has_next = PHASE > 0 || kt + 1 < KT;
        const int sn = (s + 1 == STAGES) ? 0 : s + 1;
        const int sd = (s == 0) ? STAGES - 1 : s - 1;  // buffer of stage kt+STAGES-1 (freed last stage)
        const int sac = AX ? sa : s;                    // A buffer of this stage
        const int san = AX ? ((sa + 1 == SA) ? 0 : sa + 1) : sn;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const int cur = kk & 1, nxt = cur ^ 1;
#pragma unroll
            for (int i = 0; i < NMMA; ++i) {
                mma_op(cur, i);
                const int slot = kk * NMMA + i;
                if constexpr (RING && EARLY && AX && PHASE >= 1) {
                    // B of stage kt+2 into this stage's B buffer, then (PHASE 2) A of stage kt+3 into its A buffer
                    if (slot > LAST && (slot - LAST - 1) % DSTRIDE == 0) {
                        const int q = (slot - LAST - 1) / DSTRIDE;
                        if (q < B_INS) {
                            dma_op(A_INS + q, kt + 2, sac, s);
                        } else if (PHASE == 2 && q < PER_STAGE) {
                            dma_op(q - B_INS, kt + 3, sac, s);
                        }
                    }
                } else if constexpr (RING && PHASE == 2 && EARLY && !AX) {
                    if (slot > LAST && (slot - LAST - 1) % DSTRIDE == 0 && (slot - LAST - 1) / DSTRIDE < PER_STAGE)
                        dma_op((slot - LAST - 1) / DSTRIDE, kt + STAGES, s, s);
                } else if constexpr (RING && PHASE == 2 && !AX) {
                    if (slot % DSTRIDE == 0 && slot / DSTRIDE < PER_STAGE) dma_op(slot / DSTRIDE, kt + STAGES - 1, sd, sd);
                }
                if constexpr (LOADER == LOAD_REG && PHASE >= 1) {
                    if (slot >= CSLOT && slot < CSLOT + PER_STAGE) lwrite_op(slot - CSLOT, sn);
                }
                if constexpr (LOADER == LOAD_REG && PHASE == 2) {
                    if (slot >= CSLOT && (slot - CSLOT) % DSTRIDE == 0 && (slot - CSLOT) / DSTRIDE < PER_STAGE)
                        gload_op((slot - CSLOT) / DSTRIDE, kt + 2);
                }
                if constexpr (INPLACE) {
                    if (i == 0) read_a(TM - 1, sac, kk);  // before this stage's barrier: stage s is still live
                    if (kk + 1 < KSTEPS) {
#pragma unroll
                        for (int jb = 0; jb < NB; ++jb)
                            if (read_slot<NB, BSPREAD>(jb, 0, NMMA) == i) read_b(nxt, jb, s, kk + 1);
#pragma unroll
                        for (int mi = 0; mi + 1 < TM; ++mi)
                            if ((mi + 1) * TN - 1 == i) read_a(mi, sac, kk + 1);
                    } else if (has_next) {
                        if (i == BSLOT) {
                            if constexpr (RING && AX) {
                                // stage kt+1 (A issued two stages ago, B last stage) must have landed; A of
                                // stage kt+2, issued last of all last stage (or in the prologue), may remain
                                if (kt + 2 < KT) {
                                    wait_vmcnt<A_INS>();
                                } else {
                                    wait_vmcnt0();
                                }
                            } else if constexpr (RING) {
                                if constexpr (PHASE == 2) {
                                    wait_vmcnt<(STAGES - 2) * PER_STAGE>();
                                } else {
                                    wait_vmcnt0();
                                }
                            }
                            __syncthreads();
                        }
#pragma unroll
                        for (int jb = 0; jb < NB; ++jb)
                            if (read_slot<NB, BSPREAD>(jb, BSLOT + 1, NMMA - BSLOT - 1) == i) read_b(nxt, jb, sn, 0);
#pragma unroll
                        for (int mi = 0; mi + 1 < TM; ++mi)
                            if (max((mi + 1) * TN - 1, BSLOT + 1) == i) read_a(mi, san, 0);
                    }
                } else if (kk + 1 < KSTEPS) {
#pragma unroll
                    for (int j = 0; j < NRD; ++j)
                        if (read_slot<NRD, (SPREAD & 1)>(j, 0, NMMA) == i) read_op(nxt, j, s, kk + 1);
                } else if (has_next) {
                    if (i == BSLOT) {
                        if constexpr (RING) {
                            if constexpr (PHASE == 2) {
                                wait_vmcnt<(STAGES - 2) * PER_STAGE>();
                            } else {
                                wait_vmcnt0();
                            }
                        }
                        __syncthreads();
                    }
#pragma unroll
                    for (int j = 0; j < NRD; ++j)
                        if (read_slot<NRD, (SPREAD & 1)>(j, BSLOT + 1, NMMA - BSLOT - 1) == i) read_op(nxt, j, sn, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        s = sn;
        sa = san;
    };
    // PINNED: the MFMAs are inline asm on accumulators pinned to AGPRs, so the
    // compiler inserts no MFMA hazard waits around them.  Fragments come from
    // LDS (covered by lgkmcnt waits on the asm operands), and each accumulator
    // is reused only a full k-step later.  Left to cover here: the zeroing
    // writes before the first MFMA, and the epilogue's reads of the last
    // results (16 passes + 2 for 32x32, less for 16x16).  Each accumulator
    // passes through an empty volatile asm on the near side of the s_nops,
    // which orders its writes (reads) before (after) them.
    auto pin_order = [&]() {
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni) asm volatile("" : "+a"(acc[mi][ni]));
    };
    if constexpr (PINNED) {
        pin_order();
        asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
    }
    int kt = 0;
    if constexpr (RING && AX) {
        // PHASE 2 while A of kt+3 exists, PHASE 1 (B of kt+2 only) for kt = KT-3
        for (; kt < KT - 3; ++kt) stage.template operator()<2>(kt);
        if (kt < KT - 2) stage.template operator()<1>(kt++);
    } else if constexpr (RING) {
        // PHASE 2 while the stage its copies fill exists: kt+STAGES-1 (EARLY: kt+STAGES) < KT
        for (; kt < KT - (EARLY ? STAGES : STAGES - 1); ++kt) stage.template operator()<2>(kt);
    } else {
        for (; kt < KT - 2; ++kt) stage.template operator()<2>(kt);
        if (kt < KT - 1) stage.template operator()<1>(kt++);
    }
    for (; kt < KT; ++kt) stage.template operator()<0>(kt);
    if constexpr (PINNED) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        pin_order();
    }
    stamp(2);

    // The epilogue's per-lane index math starts from a thread id that passes
    // through an empty asm here, after the K loop, so the compiler cannot
    // hoist any of it above the loop, where its registers would add to the
    // loop's (one such hoisted address once pushed a bias-epilogue kernel past
    // 256 VGPRs into a scratch spill).
    int tid_e = (int)threadIdx.x;
    asm volatile("" : "+v"(tid_e));
    const int lane_e = tid_e & 63, wave_e = tid_e >> 6;
    const int wm_e = wave_e / WN, wn_e = wave_e % WN;

    // Epilogue on the accumulators, one write of C.  Lane l holds, of block
    // (mi, ni), the 4 consecutive columns
    //   MF = 32, register 4*r4 + e: C[mi*32 + l%32][ni*32 + 8*r4 + 4*(l/32) + e]
    //   MF = 16, register e:        C[mi*16 + l%16][ni*16 + 4*(l/16) + e]
    // relative to the wave's sub-tile origin (m0 + wm*WTM, n0 + wn*WTN).
    // With LOAD_DMA, N % 8 == 0, so a column quad is all in or all out.
    //
    // LDS_EPI (SPREAD bit 5): the stage buffers are free once the last stage
    // has been read, and the whole fp16 C tile fits in them.  Each wave writes
    // its sub-tile there in the MFMA layout (8 bytes per lane, rows of WTN
    // columns whose 16-byte chunks are XOR-swizzled by row), one MFMA row
    // block at a time, and reads each block back row-contiguous and writes it
    // to C with 16-byte stores before it forms the next: one store instruction
    // covers 64 consecutive 16-byte chunks of the sub-tile's rows (RCH = WTN/8
    // chunks per row) instead of MF rows x 8 bytes x 4 lanes, and the stores
    // of a block go out while the wave forms the next ones.
    // NT_C (SPREAD bit 6): those stores are marked non-temporal (C is not
    // read again by this kernel).
    constexpr int NQ = NACC / 4;  // column quads per lane and block
    constexpr bool LDS_EPI = (SPREAD & 32) != 0;
    constexpr bool NT_C = (SPREAD & 64) != 0;
    static_assert(!NT_C || LDS_EPI, "non-temporal C stores belong to the LDS epilogue");
    constexpr int RCH = WTN / 8;                     // 16-byte chunks per sub-tile row
    constexpr bool RCH_P2 = (RCH & (RCH - 1)) == 0;
    static_assert(!LDS_EPI || (BM * BN * 2 <= Cfg::LDS_BYTES && ((RCH_P2 && RCH >= 4 && RCH <= 64) || RCH == 12)),
                  "LDS epilogue: the C tile fits in the stage buffers; 4..64 (power of two) or 12 chunks per row");
    // Chunk swizzle of sub-tile row r.  Power-of-two rows: XOR with the low row
    // bits (up to 16 rows spread over distinct bank groups).  12-chunk rows
    // (192 bytes): rows r and r + 4 start at the same bank, so XOR with bits 2-3
    // of r, which keeps a chunk inside its aligned group of 4 and so inside the row.
    auto c_swz = [&](int r) { return RCH_P2 ? (r & ((RCH < 16 ? RCH : 16) - 1)) : ((r >> 2) & 3); };
    GK_LDS char* const c_lds = a_lds + wave_e * (WTM * WTN * 2);  // this wave's sub-tile [WTM][WTN] fp16
    // C in row blocks: for each MFMA row block mi, the epilogue of its accumulators, then (LDS_EPI) its rows
    // staged through LDS and stored at once, so that a wave's C stores go out while it still forms the next
    // row blocks (rows of block mi are complete once every column block of it is written).
    auto col_of = [&](int ni, int r4) {  // column of the lane's quad in the sub-tile
        return ni * MF + (MF == 32 ? 8 * r4 + 4 * (lane_e >> 5) : 4 * (lane_e >> 4));
    };
    auto bias_quad = [&](int n, float (&bv)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = 0.0f;
        if constexpr (EPI != EPI_NONE) {
            if (n + 4 <= N) {
                const f16x4 b4 = *(const f16x4_u*)(p.bias + n);
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[e] = (float)b4[e];
            } else if (LOADER != LOAD_DMA) {  // LOAD_DMA: N % 8 == 0, the quad is wholly past N
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < N) bv[e] = (float)p.bias[n + e];
            }
        }
    };
    if constexpr (LDS_EPI) {
        __syncthreads();  // every wave has finished reading the last stage
        // 16-byte stores need 16-byte-aligned rows of C (always so with LOAD_DMA)
        const bool c_al = LOADER == LOAD_DMA || ((((uintptr_t)p.C) & 15) == 0 && (ldc & 7) == 0);
        constexpr int ITB = MF * RCH / 64;  // store instructions per row block
        static_assert((MF * RCH) % 64 == 0, "whole store instructions per row block");
        float bvs[TN][NQ][4];
#pragma unroll
        for (int ni = 0; ni < TN; ++ni)
#pragma unroll
            for (int r4 = 0; r4 < NQ; ++r4) bias_quad(n0 + wn_e * WTN + col_of(ni, r4), bvs[ni][r4]);
#pragma unroll
        for (int mi = 0; mi < TM; ++mi) {
            const int rr = mi * MF + (lane_e % MF);  // row in the sub-tile
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int r4 = 0; r4 < NQ; ++r4) {
                    const int nc = col_of(ni, r4);
                    f16x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = (f16)apply_epilogue<EPI>(acc[mi][ni][4 * r4 + e], bvs[ni][r4][e]);
                    *(GK_LDS f16x4*)(c_lds + rr * WTN * 2 + (((nc >> 3) ^ c_swz(rr)) << 4) + ((nc & 7) << 1)) = o;
                }
            // Each wave reads back only the region it wrote (its own sub-tile): once this wave's LDS writes
            // have completed, its lanes read what other lanes of the same wave wrote.  The memory clobber keeps
            // the compiler from moving the reads above the wait.
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int j = 0; j < ITB; ++j) {
                const int lc = (mi * ITB + j) * 64 + lane_e;  // chunk of the sub-tile, row-major
                const int rc = lc / RCH, c = lc % RCH;
                const f16x8 v = *(const GK_LDS f16x8*)(c_lds + rc * WTN * 2 + ((c ^ c_swz(rc)) << 4));
                const int m = m0 + wm_e * WTM + rc, n = n0 + wn_e * WTN + 8 * c;
                if (m >= M || n >= N) continue;
                f16* dst = p.C + (size_t)m * ldc + n;
                if (n + 8 <= N) {
                    if (c_al) {
                        if constexpr (NT_C) {
                            __builtin_nontemporal_store(v, (f16x8*)dst);
                        } else {
                            *(f16x8*)dst = v;
                        }
                    } else {
                        *(f16x8_u*)dst = v;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < N) dst[e] = v[e];
                }
            }
        }
    } else {
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
#pragma unroll
            for (int r4 = 0; r4 < NQ; ++r4) {
                const int nc = col_of(ni, r4);
                const int n = n0 + wn_e * WTN + nc;
                const bool quad = n + 4 <= N;
                float bv[4];
                bias_quad(n, bv);
#pragma unroll
                for (int mi = 0; mi < TM; ++mi) {
                    const int rr = mi * MF + (lane_e % MF);  // row in the sub-tile
                    f16x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = (f16)apply_epilogue<EPI>(acc[mi][ni][4 * r4 + e], bv[e]);
                    const int m = m0 + wm_e * WTM + rr;
                    if (m >= M || n >= N) continue;
                    f16* dst = p.C + (size_t)m * ldc + n;
                    if (quad) {
                        *(f16x4_u*)dst = o;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < N) dst[e] = o[e];
                    }
                }
            }
        }
    }
    if constexpr (GK_TIMELINE) {
        wait_vmcnt0();  // the C stores have completed
        stamp(3);
        if (p.timeline != nullptr && (threadIdx.x & 63) == 0) {
            uint64_t* o = p.timeline + ((size_t)blockIdx.x * (WM * WN) + (threadIdx.x >> 6)) * 8;
            o[2] = tl[2];
            o[3] = tl[3];
            o[6] = tl[6];
            o[7] = tl[7];
        }
    }
}

}  // namespace gk
