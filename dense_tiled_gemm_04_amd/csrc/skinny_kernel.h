// Skinny-M fp16 GEMM for gfx950 (M <= 16 * MB): the HBM-bound shape, where B
// is streamed exactly once and A (M x K, a few hundred KiB) stays in L2.
//
// The tutorial notes that bandwidth-bound kernels are limited by memory
// traffic rather than math (TileLang blog post, section on pitfalls; news
// article, paragraph on the fused epilogue and memory-bandwidth bottlenecks).
// Here the design goal is to keep enough bytes of B in flight per CU:
//  * one workgroup = 4 wave64s owns a 64-column panel of B/C and all of K;
//    the grid has ceil(N / 64) workgroups (256 for N = 16384: one per CU);
//  * B and A reach LDS by asynchronous LDS-DMA (buffer_load ... lds), STAGES
//    deep, so the bytes in flight do not occupy VGPRs; B, read exactly once,
//    is loaded non-temporal;
//  * B rows past K fall outside the buffer range and read as zero, which
//    zeroes a ragged K tail without per-lane masks; A rows are range-masked
//    at the same granularity (see below);
//  * wave w computes the 16-column block w of the panel with
//    v_mfma_f32_16x16x32_f16, B fragments via the LDS transpose read;
//  * the fused epilogue runs on the accumulators; C is written once.
// With B given transposed (Bt[N][K], a linear layer's weight) the panel is
// 64 rows of Bt, k-contiguous: its stage is laid out and read like A's (one
// 16-byte LDS read per fragment instead of two transpose reads), and k-chunks
// past K are sent out of range as A's are.
// A16: A reaches LDS by 16-byte LDS-DMA (one or a few copies per lane and
// stage) instead of 4-byte copies (four times as many).  K % 8 == 0 on this
// path, so a 16-byte chunk of A never straddles K; chunks past K are sent out
// of range like single dwords.
// KROT: workgroup w walks its K stages starting at stage w mod KT (wrapping
// around).  With Bt, the workgroups' concurrent reads then sit at different
// offsets within their rows instead of all at the same one, 16 KiB apart,
// which spreads them over the HBM channels.  Only the fp32 summation order of
// each column changes.
#pragma once
#include "common.h"

namespace gk {

constexpr int SK_BN = 64;       // panel width (columns of B / C per workgroup)
constexpr int SK_BK = 128;      // K rows per stage
constexpr int SK_WAVES = 4;

// B stage: [SK_BK][SK_BN] fp16, 8 chunks of 16 bytes per row.  Logical chunk
// c of row kr lives at c ^ sk_swz_b(kr); a half-wave transpose read touches
// 8 rows x 2 chunks, which this spreads over 16 distinct bank groups.
__device__ __forceinline__ int sk_swz_b(int kr) {
    return 2 * (((kr >> 1) & 1) | (((kr >> 3) & 1) << 1));
}

template <int MB, int STAGES, int EPI, int BT, int KROT, int A16>
__global__ void __launch_bounds__(SK_WAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
gemm_skinny_kernel(GemmArgs p) {
    constexpr int NT = SK_WAVES * 64;
    constexpr int MR = 16 * MB;                      // A rows held per stage
    constexpr int B_STAGE = SK_BK * SK_BN * 2;       // 16 KiB
    constexpr int A_STAGE = MR * SK_BK * 2;          // 4 KiB per 16 rows
    constexpr int B_INS = B_STAGE / 16 / NT;         // 16-byte DMA per lane
    constexpr int A_BYTES = A16 ? 16 : 4;            // bytes per A copy and lane
    constexpr int A_INS = A_STAGE / A_BYTES / NT;    // A copies per lane
    static_assert(B_INS * 16 * NT == B_STAGE && A_INS * A_BYTES * NT == A_STAGE, "stage split");
    __shared__ __attribute__((aligned(1024))) char smem_raw[STAGES * (A_STAGE + B_STAGE)];
    GK_LDS char* smem = (GK_LDS char*)smem_raw;
    GK_LDS char* const b_lds = smem;
    GK_LDS char* const a_lds = smem + STAGES * B_STAGE;

    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb, ldc = p.ldc;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * SK_BN;
    const int KT = (K + SK_BK - 1) / SK_BK;

    // Buffer resources: B ends with its last row (element (K-1)*ldb + N), so
    // k-rows >= K read 0; A ends with its last row, and so does Bt.
    const int64_t b_elems = BT ? (int64_t)(N - 1) * ldb + K : (int64_t)(K - 1) * ldb + N;
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.B, (short)0, (int)min(b_elems * 2, (int64_t)0x7fffffff), 0x00020000);
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.A, (short)0, (int)min(((int64_t)(M - 1) * lda + K) * 2, (int64_t)0x7fffffff), 0x00020000);

    // Per-lane DMA source offsets within one stage.
    uint32_t b_off[B_INS];
    int b_kc[B_INS];  // BT: k offset of the chunk within the stage
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        const int P = (i * SK_WAVES + wave) * 64 + lane;  // destination chunk in the stage
        if constexpr (BT) {
            // Bt stage: [SK_BN][SK_BK], 16 chunks per row, chunk c of row r at c ^ (r & 15);
            // rows past N re-read row N-1 (their columns are never stored)
            const int r = P >> 4, c = (P & 15) ^ (r & 15);
            b_kc[i] = 8 * c;
            b_off[i] = (uint32_t)(((int64_t)min(n0 + r, N - 1) * ldb + 8 * c) * 2);
        } else {
            const int kr = P >> 3, pc = P & 7;
            const int c = pc ^ sk_swz_b(kr);
            const int n = min(n0 + 8 * c, N - 8);          // past-N columns re-read the last chunk
            b_off[i] = (uint32_t)((kr * ldb + n) * 2);
            b_kc[i] = 0;
        }
    }
    // A stage: [MR][SK_BK] fp16 = 16 chunks per row, chunk c of row m at c ^ (m & 15).
    // Rows >= M are clamped to M-1 (results never stored); a copy past K in a
    // row would read the next row's data, multiplied by B rows that read as
    // zero.  That product is 0 for finite A; to keep it exact even for
    // non-finite A, copies past K are redirected out of range (read as 0) below.
    uint32_t a_off[A_INS];
    int a_kcol[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        int m, c, w;
        if constexpr (A16) {
            const int P = (i * SK_WAVES + wave) * 64 + lane;   // destination chunk in the stage
            m = P >> 4;
            c = (P & 15) ^ (m & 15);
            w = 0;
        } else {
            const int D = (i * SK_WAVES + wave) * 64 + lane;   // destination dword in the stage
            m = D >> 6;
            c = ((D >> 2) & 15) ^ (m & 15);
            w = D & 3;
        }
        const int mm = min(m, M - 1);
        a_kcol[i] = 8 * c + 2 * w;                             // k offset within the stage
        a_off[i] = (uint32_t)((mm * lda + a_kcol[i]) * 2);
    }

    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t b_lds0 = lds_addr(b_lds) + wave_s * 64 * 16;
    const uint32_t a_lds0 = lds_addr(a_lds) + wave_s * 64 * A_BYTES;
    const int krot = (KROT && KT > 0) ? (int)(blockIdx.x % (unsigned)KT) : 0;
    auto issue = [&](int kt, int s) {
        const int ktr = kt + krot < KT ? kt + krot : kt + krot - KT;
        const int kbase = ktr * SK_BK;
#pragma unroll
        for (int i = 0; i < B_INS; ++i) {
            uint32_t off;
            if constexpr (BT) {  // k-chunks past K (K % 8 == 0) read as zero
                off = (kbase + b_kc[i] < K) ? b_off[i] + (uint32_t)kbase * 2 : 0x80000000u;
            } else {
                off = b_off[i] + (uint32_t)kbase * ldb * 2;
            }
            dma_buffer_16_nt(b_rsrc, off, b_lds0 + s * B_STAGE + i * SK_WAVES * 64 * 16);
        }
#pragma unroll
        for (int i = 0; i < A_INS; ++i) {
            const uint32_t off = (kbase + a_kcol[i] < K) ? a_off[i] + (uint32_t)kbase * 2 : 0x80000000u;
            if constexpr (A16) {
                dma_buffer_16(a_rsrc, off, a_lds0 + s * A_STAGE + i * SK_WAVES * 64 * 16);
            } else {
                dma_buffer_4(a_rsrc, off, a_lds0 + s * A_STAGE + i * SK_WAVES * 64 * 4);
            }
        }
    };

    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // MFMA 16x16x32 as D[n][m] = B^T . A^T:
    //  operand a (B^T): lane l holds B[k = 8*(l/16) + 0..7][n = l%16], built from
    //   two transpose reads; lane L = 16g + 4j + q addresses B[8g + 4h + j][4q..4q+3];
    //  operand b (A^T): lane l holds A[m = l%16][k = 8*(l/16) + 0..7].
    auto compute_stage = [&](int s) {
        const GK_LDS char* Bs = b_lds + s * B_STAGE;
        const GK_LDS char* As = a_lds + s * A_STAGE;
        const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
        const int nl = wave * 16 + 4 * q;                  // column within the panel
#pragma unroll
        for (int ks = 0; ks < SK_BK / 32; ++ks) {
            f16x8 bf;
            if constexpr (BT) {  // lane l: Bt[n = 16 wave + l%16][k = 32 ks + 8 (l/16) .. +7]
                const int r = wave * 16 + (lane & 15);
                bf = *(const GK_LDS f16x8*)(Bs + r * SK_BK * 2 + (((4 * ks + g) ^ (r & 15)) << 4));
            } else {
                f16x4 half_[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kr = 32 * ks + 8 * g + 4 * h + j;
                    const int c = (nl >> 3) ^ sk_swz_b(kr);
                    half_[h] = lds_read_tr16_b64(Bs + kr * SK_BN * 2 + (c << 4) + ((nl & 7) << 1));
                }
                bf = __builtin_shufflevector(half_[0], half_[1], 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int m = 16 * mb + (lane & 15);
                const int c = (4 * ks + g) ^ (m & 15);
                const f16x8 af = *(const GK_LDS f16x8*)(As + m * SK_BK * 2 + (c << 4));
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, af, acc[mb], 0, 0, 0);
            }
        }
    };
    // Pipeline: STAGES-1 stages in flight.  Every wave issues B_INS + A_INS
    // DMA instructions per stage, and vector-memory loads complete in order,
    // so "stage kt has landed" is vmcnt <= (stages issued after it) * per-stage.
    constexpr int PER_STAGE = B_INS + A_INS;
    static_assert((STAGES - 2) * PER_STAGE <= 63, "vmcnt range");
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < KT) issue(s, s);
    for (int kt = 0; kt < KT; ++kt) {
        const int after = min(KT - 1 - kt, STAGES - 2);    // stages issued after kt
        if (after >= STAGES - 2) {
            wait_vmcnt<(STAGES - 2) * PER_STAGE>();
        } else {
            wait_vmcnt0();
        }
        __syncthreads();
        if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
        compute_stage(kt % STAGES);
    }

    // Epilogue.  Lane l, register r of block mb holds C[16*mb + l%16][n0 + 16*wave + 4*(l/16) + r].
    const int n = n0 + wave * 16 + 4 * (lane >> 4);
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (EPI != EPI_NONE) {
        if (n + 4 <= N) {
            f16x4 b4 = *(const f16x4*)(p.bias + n);
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[e] = (float)b4[e];
        }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = 16 * mb + (lane & 15);
        if (m < M && n + 4 <= N) {
            f16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (f16)apply_epilogue<EPI>(acc[mb][e], bv[e]);
            *(f16x4*)(p.C + (size_t)m * ldc + n) = o;
        }
    }
}

}  // namespace gk
