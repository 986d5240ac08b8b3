// Split-K form of the skinny-M fp16 GEMM (M <= 16 * MB, B[K][N] row-major):
// two kernels on one stream, deterministic, with no inter-workgroup fences.
//
// The tutorial notes that bandwidth-bound kernels are limited by memory
// traffic rather than math (TileLang blog post, section on pitfalls; news
// article, paragraph on the fused epilogue and memory-bandwidth bottlenecks).
// B (K x N) is read exactly once either way; what changes is the shape of the
// reads.  The one-pass skinny kernel gives each workgroup a 64-column panel
// (128-byte row segments, 32 KiB apart for N = 16384) over all of K.  Here a
// workgroup takes a 256-column panel (512-byte segments) over one of S
// contiguous K ranges, so the same 256 workgroups read four times longer
// segments:
//  * pass 1 (gemm_skinny_splitk_kernel): workgroup (panel p, range s) streams
//    B rows [s*KC, min(K, (s+1)*KC)) x columns [256 p, 256 p + 256) through an
//    LDS-DMA ring (non-temporal: read once), multiplies by the matching A
//    columns with v_mfma_f32_16x16x32_f16 and writes its fp32 partial sums
//    P[s][m][n], 16-byte stores;
//  * pass 2 (splitk_reduce_kernel): C[m][n] = epi(P[0][m][n] + ... + P[S-1][m][n]
//    + bias[n]), summed in increasing s, then rounded once to fp16.
// The sum over k is therefore taken in fp32 in a fixed order: in k order within
// a range, then over the ranges in order.  The stream orders pass 2 after
// pass 1; no atomics, counters or cross-workgroup waits.
#pragma once
#include "common.h"
#include "tile_pipe_kernel.h"

namespace gk {

constexpr int SKS_BN = 256;     // panel width (columns of B / C per workgroup)
constexpr int SKS_WAVES = 4;    // each wave owns 64 columns of the panel

template <int MB, int STAGES, int BK>
__global__ void __launch_bounds__(SKS_WAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
gemm_skinny_splitk_kernel(GemmArgs p) {
    constexpr int NT = SKS_WAVES * 64;
    constexpr int MR = 16 * MB;                        // A rows held per stage
    constexpr int CB = SKS_BN / 8;                     // 16-byte chunks per B row (32)
    constexpr int CA = BK / 8;                         // 16-byte chunks per A row
    constexpr int B_STAGE = BK * SKS_BN * 2;
    constexpr int A_STAGE = MR * BK * 2;
    constexpr int B_INS = B_STAGE / 16 / NT;           // 16-byte copies per lane and stage
    constexpr int A_INS = A_STAGE / 4 / NT;            // 4-byte copies per lane and stage
    constexpr int PER_STAGE = B_INS + A_INS;
    constexpr int TN = 64 / 16;                        // 16-column MFMA blocks per wave
    static_assert(BK % 32 == 0 && B_INS * 16 * NT == B_STAGE && A_INS * 4 * NT == A_STAGE, "stage split");
    static_assert(STAGES >= 2 && (STAGES - 2) * PER_STAGE <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char smem_raw[STAGES * (A_STAGE + B_STAGE)];
    GK_LDS char* const b_lds = (GK_LDS char*)smem_raw;
    GK_LDS char* const a_lds = b_lds + STAGES * B_STAGE;

    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int panel = (int)blockIdx.x % p.tiles_n, split = (int)blockIdx.x / p.tiles_n;
    const int n0 = panel * SKS_BN;
    const int k_lo = split * p.k_chunk;
    const int KT = k_lo < K ? (min(K, k_lo + p.k_chunk) - k_lo + BK - 1) / BK : 0;  // stages of this range

    // Buffer resources from the start of B and A to the end of their last rows: B rows at or past K read 0
    // (only the last range can reach them), A chunks at or past K are sent out of range below.
    const int64_t b_elems = (int64_t)(K - 1) * ldb + N;
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.B, (short)0, (int)min(b_elems * 2, (int64_t)0x7fffffff), 0x00020000);
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.A, (short)0, (int)min(((int64_t)(M - 1) * lda + K) * 2, (int64_t)0x7fffffff), 0x00020000);

    // B stage [BK][256]: destination chunk P = (i * 4 + wave) * 64 + lane holds logical chunk
    // c = (P % CB) ^ swz_b(kr) of k-row kr = P / CB.  Columns past N are never stored; with N % 8 == 0 a
    // chunk is wholly in or out, and one past N reads the next row (or zeros past the end of B).
    uint32_t b_off[B_INS];
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        const int P = (i * SKS_WAVES + wave) * 64 + lane;
        const int kr = P / CB, c = (P % CB) ^ swz_b<SKS_BN, 16>(kr);
        b_off[i] = (uint32_t)((kr * ldb + n0 + 8 * c) * 2);
    }
    // A stage [MR][BK], dword copies: destination dword D = (i * 4 + wave) * 64 + lane, row m = D / (BK / 2),
    // physical chunk D % (BK / 2) / 4 holding logical chunk c = physical ^ swz_a(m), dword w within it.
    // Rows past M re-read row M-1 (never stored).
    uint32_t a_off[A_INS];
    int a_k[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int D = (i * SKS_WAVES + wave) * 64 + lane;
        const int m = D / (BK / 2), dw = D % (BK / 2);
        const int c = (dw >> 2) ^ swz_a<BK>(m), w = dw & 3;
        a_k[i] = 8 * c + 2 * w;
        a_off[i] = (uint32_t)((min(m, M - 1) * lda + a_k[i]) * 2);
    }

    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t b_lds0 = lds_addr(b_lds) + wave_s * 64 * 16;
    const uint32_t a_lds0 = lds_addr(a_lds) + wave_s * 64 * 4;
    auto issue = [&](int kt, int s) {
        const int kbase = k_lo + kt * BK;
#pragma unroll
        for (int i = 0; i < B_INS; ++i)
            dma_buffer_16_nt(b_rsrc, b_off[i] + (uint32_t)kbase * ldb * 2, b_lds0 + s * B_STAGE + i * NT * 16);
#pragma unroll
        for (int i = 0; i < A_INS; ++i) {
            const uint32_t off = kbase + a_k[i] < K ? a_off[i] + (uint32_t)kbase * 2 : 0x80000000u;
            dma_buffer_4(a_rsrc, off, a_lds0 + s * A_STAGE + i * NT * 4);
        }
    };

    f32x4 acc[MB][TN];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) acc[mb][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

    // MFMA 16x16x32 as D[n][m] = B^T . A^T.  Operand a (B^T): lane l holds B[k = 8 (l/16) .. +7][n = l%16]
    // of the block, from two transpose reads; lane L = 16 g + 4 j + q addresses k-row 8 g + 4 h + j and
    // columns 4q .. 4q+3.  Operand b (A^T): lane l holds A[m = l%16][k = 8 (l/16) .. +7].
    const int g4 = lane >> 4, jj = (lane >> 2) & 3, q = lane & 3;
    int b_rd[TN];
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
        const int kr = 8 * g4 + jj;
        const int nl = wave * 64 + ni * 16 + 4 * q;
        b_rd[ni] = kr * SKS_BN * 2 + (((nl >> 3) ^ swz_b<SKS_BN, 16>(kr)) << 4) + ((nl & 7) << 1);
    }
    auto compute_stage = [&](int s) {
        const GK_LDS char* Bs = b_lds + s * B_STAGE;
        const GK_LDS char* As = a_lds + s * A_STAGE;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            f16x8 af[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int m = 16 * mb + (lane & 15);
                af[mb] = *(const GK_LDS f16x8*)(As + m * BK * 2 + (((4 * ks + g4) ^ swz_a<BK>(m)) << 4));
            }
#pragma unroll
            for (int ni = 0; ni < TN; ++ni) {
                // the swizzle of k-row kr depends on bits 0, 1 and 3 only: + 4 h and + 32 ks leave it unchanged
                const f16x4 h0 = lds_read_tr16_b64(Bs + b_rd[ni] + (32 * ks) * SKS_BN * 2);
                const f16x4 h1 = lds_read_tr16_b64(Bs + b_rd[ni] + (32 * ks + 4) * SKS_BN * 2);
                const f16x8 bf = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb][ni] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, af[mb], acc[mb][ni], 0, 0, 0);
            }
        }
    };

    // Ring of STAGES buffers, STAGES-1 stages in flight; every wave issues PER_STAGE copies per stage and
    // vector-memory operations complete in order, so "stage kt has landed" is vmcnt <= copies issued after it.
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < KT) issue(s, s);
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + STAGES - 2 < KT) {
            wait_vmcnt<(STAGES - 2) * PER_STAGE>();
        } else {
            wait_vmcnt0();
        }
        __syncthreads();
        if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
        compute_stage(kt % STAGES);
    }

    // Partial sums: lane l, register e of block (mb, ni) holds the sum for
    // C[16 mb + l%16][n0 + 64 wave + 16 ni + 4 (l/16) + e] over this range (zero for an empty range).
    float* const P = p.partial + (size_t)split * M * N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = 16 * mb + (lane & 15);
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            const int n = n0 + wave * 64 + ni * 16 + 4 * (lane >> 4);
            if (m < M && n < N) *(f32x4*)(P + (size_t)m * N + n) = acc[mb][ni];
        }
    }
}

// C[m][n] = epi(sum over s of P[s][m][n], bias[n]), 4 consecutive columns per thread (N % 8 == 0).  The
// `splits` ranges (at most S) are loaded together and summed in increasing s.
template <int EPI, int S>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(GemmArgs p) {
    const int M = p.M, N = p.N, splits = p.k_split;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)M * (N / 4)) return;
    const int m = (int)(idx / (N / 4)), n = (int)(idx % (N / 4)) * 4;
    f32x4 v[S];
#pragma unroll
    for (int sp = 0; sp < S; ++sp)
        v[sp] = sp < splits ? *(const f32x4*)(p.partial + ((size_t)sp * M + m) * N + n) : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 sum = v[0];
#pragma unroll
    for (int sp = 1; sp < S; ++sp)
        if (sp < splits) sum += v[sp];
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (EPI != EPI_NONE) {
        const f16x4 b4 = *(const f16x4*)(p.bias + n);  // 8-byte aligned
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = (float)b4[e];
    }
    f16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (f16)apply_epilogue<EPI>(sum[e], bv[e]);
    *(f16x4*)(p.C + (size_t)m * p.ldc + n) = o;
}

}  // namespace gk
