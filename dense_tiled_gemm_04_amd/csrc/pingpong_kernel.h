// Ping-pong tile kernel of the fp16 GEMM on gfx950: the same product, tile and
// epilogue as gemm_tile_pipe_kernel's eight-wave 256x256 configurations, with
// a different schedule.
//
// The tutorial's tiled GEMM (blog post "Designing High-Performance GPU Kernels
// with TileLang", section "Step 4"; news article on TileLang kernel design,
// paragraphs on the tiled GEMM and the fused epilogue): fp16 tiles of A and B
// staged in shared memory, fp32 accumulators in registers, a pipelined K loop,
// bias and GELU on the accumulators before the single write of C.
//
// Schedule.  The workgroup's 8 waves form two groups of four, one wave of each
// group per SIMD: group 0 owns rows 0-127 of the 256x256 tile, group 1 rows
// 128-255, and wave wn of a group the 64 columns 64 wn .. 64 wn + 63, i.e. a
// 128x64 sub-tile of 8x4 v_mfma_f32_16x16x32_f16 blocks with its 128 fp32
// accumulators pinned to AGPRs.  Time runs in phases separated by workgroup
// barriers.  In every phase one group computes and the other loads:
//   computing: the 32 MFMAs of one 32-deep k-step, back to back, from
//              fragments already in registers;
//   loading:   the LDS reads of its next k-step's fragments (8 A reads and
//              8 B transpose reads, or 4 B reads with B transposed) and its
//              share of the global -> LDS copies, then a wait for the reads.
// Group 0 loads k-step u in phase 2u and computes it in phase 2u + 1; group 1
// does both one phase later.  So on each SIMD one wave keeps the matrix core
// busy while the other waits on LDS, and each wave needs one fragment set.
//
// LDS holds a ring of 4 slots, each a 32-deep k-slice of the A tile [256][32]
// and of the B tile [32][256] (Bt: [256][32]), 32 KiB per slot, 128 KiB in
// all.  Slot u mod 4 holds k-step u; it is read in phases 2u and 2u + 1 and is
// free after the barrier that ends phase 2u + 1.  The copies of k-step u + 3
// (into the slot of k-step u - 1) are issued by the loading group: A's by
// group 0 in phase 2u, B's by group 1 in phase 2u + 1, four 16-byte LDS-DMA
// copies per lane each.  Before the barrier that ends phase 2v - 1, after
// which group 0 reads k-step v, every wave waits until its copies of k-step v
// have landed; its copies of k-steps v + 1 and v + 2 may still be in flight.
// Copies get five phases or more to land.
//
// Copy layout, swizzles and the epilogue are those of gemm_tile_pipe_kernel
// with a 32-deep K block: XOR-swizzled 16-byte chunks (bank-conflict-free
// ds_read_b128 and ds_read_b64_tr_b16), rows past M and columns past N
// clamped on load and never stored, and the C tile staged through the freed
// slots and written with row-contiguous 16-byte stores (non-temporal with NT).
// Requires what LOAD_DMA requires with BK = 32: K % 32 == 0, N % 8 == 0,
// 16-byte-aligned rows of A, B and C and an 8-byte-aligned bias.
#pragma once
#include "common.h"
#include "tile_pipe_kernel.h"

namespace gk {

constexpr int PP_BM = 256, PP_BN = 256, PP_BK = 32, PP_SLOTS = 4, PP_WAVES = 8;
constexpr int PP_SLOT_A = PP_BM * PP_BK * 2;   // 16 KiB
constexpr int PP_SLOT_B = PP_BK * PP_BN * 2;   // 16 KiB
constexpr int PP_LDS_BYTES = PP_SLOTS * (PP_SLOT_A + PP_SLOT_B);

template <int GROUP_M, int EPI, int BT, int NT_C>
__global__ void __launch_bounds__(PP_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_pingpong_kernel(GemmArgs p) {
    constexpr int BM = PP_BM, BN = PP_BN, BK = PP_BK, MF = 16, KS = 32;
    constexpr int WN = 4, WTM = 128, WTN = 64, TM = WTM / MF, TN = WTN / MF;  // 8 x 4 MFMA blocks per wave
    constexpr int CA = BK / 8, CB = BN / 8;                                    // 16-byte chunks per row
    constexpr int NCOPY = 4;                                                   // copies per lane per k-step
    static_assert(PP_LDS_BYTES <= 160 * 1024 && BM * BN * 2 <= PP_LDS_BYTES, "LDS budget; C tile fits the slots");
    static_assert(BM * CA == NCOPY * 4 * 64 && (BT ? BN * CA : BK * CB) == NCOPY * 4 * 64, "one group copies a slot");

    __shared__ __attribute__((aligned(1024))) char smem_raw[PP_LDS_BYTES];
    GK_LDS char* const a_lds = (GK_LDS char*)smem_raw;                 // [SLOTS][BM][BK]
    GK_LDS char* const b_lds = a_lds + PP_SLOTS * PP_SLOT_A;           // [SLOTS][BK][BN] (Bt: [SLOTS][BN][BK])

    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb, ldc = p.ldc;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);          // 0: rows 0-127, 1: rows 128-255
    const int wl = __builtin_amdgcn_readfirstlane(wave & 3);            // wave within the group
    int tm, tn;
    {
        const int nwg = p.tiles_m * p.tiles_n;
        grouped_tile<GROUP_M>(xcd_contiguous_id((int)blockIdx.x, nwg), p.tiles_m, p.tiles_n, tm, tn);
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int KT = K / BK;  // k-steps (K % 32 == 0, host-checked)

    // Fragment read offsets (bytes within a slot), as in gemm_tile_pipe_kernel with BK = 32.
    const int a_rd = [&] {
        const int row = grp * WTM + (lane % MF);
        return row * BK * 2 + (((lane / MF) ^ swz_a<BK>(row)) << 4);
    }();
    int b_rd[BT ? 1 : TN];
    int bt_rd = 0;
    if constexpr (!BT) {
        const int g4 = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
        const int kr = 8 * g4 + j;
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            const int nl = wl * WTN + ni * MF + 4 * q;
            b_rd[ni] = kr * BN * 2 + (((nl >> 3) ^ swz_b<BN, MF>(kr)) << 4) + ((nl & 7) << 1);
        }
    } else {
        const int row = wl * WTN + (lane % MF);
        bt_rd = row * BK * 2 + (((lane / MF) ^ swz_a<BK>(row)) << 4);
    }

    // Copy sources.  Group 0 copies A, group 1 copies B (or Bt); copy j of wave wl fills destination chunk
    // P = (4 j + wl) * 64 + lane of the slot's tile, whose source is the logical chunk the swizzle puts at P.
    uint32_t c_off[NCOPY];
#pragma unroll
    for (int j = 0; j < NCOPY; ++j) {
        const int P = (j * 4 + wl) * 64 + lane;
        if (grp == 0 || BT) {  // rows of A (or of Bt): [256][32], CA chunks per row
            const int r = P / CA, c = (P % CA) ^ swz_a<BK>(r);
            if (grp == 0) {
                c_off[j] = (uint32_t)(((min(m0 + r, M - 1) - m0) * lda + 8 * c) * 2);
            } else {
                c_off[j] = (uint32_t)(((min(n0 + r, N - 1) - n0) * ldb + 8 * c) * 2);
            }
        } else {                // k-rows of B: [32][256], CB chunks per row, columns past N clamped
            const int kr = P / CB, c = (P % CB) ^ swz_b<BN, MF>(kr);
            c_off[j] = (uint32_t)((kr * ldb + min(n0 + 8 * c, N - 8) - n0) * 2);
        }
    }
    const char* const a_row0 = (const char*)(p.A + (size_t)m0 * lda);
    const char* const b_col0 = (const char*)(BT ? p.B + (size_t)n0 * ldb : p.B + n0);
    const uint32_t lds_dst0 = (grp == 0 ? lds_addr(a_lds) : lds_addr(b_lds)) + wl * 64 * 16;
    const int slot_bytes = grp == 0 ? PP_SLOT_A : PP_SLOT_B;
    // this wave's copies of k-step v into slot v mod 4
    auto copy = [&](int v) {
        const char* src = grp == 0 || BT ? (grp == 0 ? a_row0 : b_col0) + (size_t)v * BK * 2
                                         : b_col0 + (size_t)v * BK * ldb * 2;
        const uint32_t dst = lds_dst0 + (v & (PP_SLOTS - 1)) * slot_bytes;
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) dma_global_16(src, c_off[j], dst + j * 4 * 64 * 16);
    };
    // wait until this wave's copies of k-step v have landed; those of v + 1 and v + 2 (if any) may remain
    auto wait_copies = [&](int v) {
        if (v >= KT) return;
        const int later = (v + 1 < KT) + (v + 2 < KT);
        if (later == 2) {
            wait_vmcnt<2 * NCOPY>();
        } else if (later == 1) {
            wait_vmcnt<NCOPY>();
        } else {
            wait_vmcnt0();
        }
    };

    constexpr int NACC = 4;
    typedef float accv __attribute__((ext_vector_type(NACC)));
    accv acc[TM][TN];
#pragma unroll
    for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) acc[mi][ni] = accv{0.f, 0.f, 0.f, 0.f};
    f16x8 fa[TM];
    f16x4 fb[BT ? 1 : TN][2];
    f16x8 fbt[BT ? TN : 1];

    auto load_frags = [&](int u) {
        const int s = u & (PP_SLOTS - 1);
        const GK_LDS char* As = a_lds + s * PP_SLOT_A;
        const GK_LDS char* Bs = b_lds + s * PP_SLOT_B;
        // B first: the MFMA order below runs over ni fastest
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            if constexpr (BT) {
                fbt[ni] = *(const GK_LDS f16x8*)(Bs + bt_rd + ni * MF * BK * 2);
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) fb[ni][h] = lds_read_tr16_b64(Bs + b_rd[ni] + 4 * h * BN * 2);
            }
        }
#pragma unroll
        for (int mi = 0; mi < TM; ++mi) fa[mi] = *(const GK_LDS f16x8*)(As + a_rd + mi * MF * BK * 2);
    };
    // The 32 MFMAs of a k-step, issued only when `go` is nonzero.  The test and the branch sit inside the asm
    // blocks, so to the compiler the accumulators are updated in place on every path: a branch around them in
    // the source would join two versions of all 128 accumulators, which the register allocator copies and
    // spills.  Each block takes two A rows (8 MFMAs).
    auto mfma_all = [&](int go) {
        f16x8 b[TN];
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            if constexpr (BT) {
                b[ni] = fbt[ni];
            } else {
                b[ni] = __builtin_shufflevector(fb[ni][0], fb[ni][1], 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
#pragma unroll
        for (int mp = 0; mp < TM; mp += 2) {
            asm volatile(
                "s_cmp_eq_u32 %[go], 0\n\t"
                "s_cbranch_scc1 .Lpp_skip%=\n\t"
                "v_mfma_f32_16x16x32_f16 %[c0], %[b0], %[a0], %[c0]\n\t"
                "v_mfma_f32_16x16x32_f16 %[c1], %[b1], %[a0], %[c1]\n\t"
                "v_mfma_f32_16x16x32_f16 %[c2], %[b2], %[a0], %[c2]\n\t"
                "v_mfma_f32_16x16x32_f16 %[c3], %[b3], %[a0], %[c3]\n\t"
                "v_mfma_f32_16x16x32_f16 %[d0], %[b0], %[a1], %[d0]\n\t"
                "v_mfma_f32_16x16x32_f16 %[d1], %[b1], %[a1], %[d1]\n\t"
                "v_mfma_f32_16x16x32_f16 %[d2], %[b2], %[a1], %[d2]\n\t"
                "v_mfma_f32_16x16x32_f16 %[d3], %[b3], %[a1], %[d3]\n"
                ".Lpp_skip%=:"
                : [c0] "+a"(acc[mp][0]), [c1] "+a"(acc[mp][1]), [c2] "+a"(acc[mp][2]), [c3] "+a"(acc[mp][3]),
                  [d0] "+a"(acc[mp + 1][0]), [d1] "+a"(acc[mp + 1][1]), [d2] "+a"(acc[mp + 1][2]),
                  [d3] "+a"(acc[mp + 1][3])
                : [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]), [a0] "v"(fa[mp]),
                  [a1] "v"(fa[mp + 1]), [go] "s"(go)
                : "scc");
        }
    };
    static_assert(TN == 4 && TM % 2 == 0, "the MFMA blocks are written for 4 column blocks and pairs of rows");
    // The MFMAs are inline asm on AGPR-pinned accumulators: the compiler inserts no hazard waits around them.
    // Left to cover: the zeroing writes before the first MFMA and the epilogue's reads after the last one;
    // each accumulator passes through an empty asm on the near side of the s_nops, ordering it.
    auto pin_order = [&]() {
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni) asm volatile("" : "+a"(acc[mi][ni]));
    };
    pin_order();
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");

    // Prologue: k-steps 0, 1 and 2 in flight; k-step 0 landed everywhere before phase 0.
    for (int v = 0; v < 3; ++v)
        if (v < KT) copy(v);
    wait_copies(0);
    __syncthreads();

    // Phases t = 0 .. 2 KT, one barrier after each.  In phase t a wave of group g is s = t - g phases into its
    // own sequence: s even loads k-step s/2 (and copies k-step s/2 + 3), s odd computes k-step (s-1)/2.  One
    // code path serves both groups, so the accumulators and fragments have a single home in registers.
    // At odd t = 2u + 1 every wave waits for its copies of k-step u + 1 before the barrier.
    for (int t = 0; t <= 2 * KT; ++t) {
        const int st = t - grp;
        const bool loading = st >= 0 && (st & 1) == 0 && (st >> 1) < KT;
        const int computing = st >= 0 && (st & 1) == 1;  // k-step (st - 1) / 2 < KT, as st <= 2 KT - grp
        if (loading) {
            const int u = st >> 1;
            if (u + 3 < KT) copy(u + 3);
            load_frags(u);
        }
        mfma_all(__builtin_amdgcn_readfirstlane(computing));
        if (t & 1) wait_copies((t >> 1) + 1);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    pin_order();

    // Epilogue (as gemm_tile_pipe_kernel's LDS-staged one).  The per-lane index math starts from a thread id
    // passed through an empty asm after the K loop, so none of it is hoisted into the loop's registers.
    int tid_e = (int)threadIdx.x;
    asm volatile("" : "+v"(tid_e));
    const int lane_e = tid_e & 63, wave_e = tid_e >> 6;
    const int wm_e = wave_e >> 2, wn_e = wave_e & 3;
    // Lane l holds, of block (mi, ni), the 4 consecutive columns C[mi*16 + l%16][ni*16 + 4*(l/16) + e]
    // of the wave's sub-tile (origin m0 + 128 wm, n0 + 64 wn).
    constexpr int RCH = WTN / 8;  // 8 chunks of 16 bytes per sub-tile row
    auto c_swz = [&](int r) { return r & (RCH - 1); };
    GK_LDS char* const c_lds = a_lds + wave_e * (WTM * WTN * 2);  // this wave's sub-tile [128][64] fp16
    __syncthreads();  // every wave has finished reading the slots (and the other group its last MFMAs' inputs)
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
        const int nc = ni * MF + 4 * (lane_e >> 4);
        const int n = n0 + wn_e * WTN + nc;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (EPI != EPI_NONE) {
            if (n + 4 <= N) {  // N % 8 == 0: a column quad is all in or all out
                const f16x4 b4 = *(const f16x4*)(p.bias + n);
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[e] = (float)b4[e];
            }
        }
#pragma unroll
        for (int mi = 0; mi < TM; ++mi) {
            const int rr = mi * MF + (lane_e % MF);
            f16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (f16)apply_epilogue<EPI>(acc[mi][ni][e], bv[e]);
            *(GK_LDS f16x4*)(c_lds + rr * WTN * 2 + (((nc >> 3) ^ c_swz(rr)) << 4) + ((nc & 7) << 1)) = o;
        }
    }
    __syncthreads();  // the sub-tile's LDS writes precede its reads by other lanes
#pragma unroll
    for (int it = 0; it < WTM * RCH / 64; ++it) {
        const int lc = it * 64 + lane_e;
        const int rr = lc / RCH, c = lc % RCH;
        const f16x8 v = *(const GK_LDS f16x8*)(c_lds + rr * WTN * 2 + ((c ^ c_swz(rr)) << 4));
        const int m = m0 + wm_e * WTM + rr, n = n0 + wn_e * WTN + 8 * c;
        if (m >= M || n >= N) continue;
        f16* dst = p.C + (size_t)m * ldc + n;
        if constexpr (NT_C) {
            __builtin_nontemporal_store(v, (f16x8*)dst);
        } else {
            *(f16x8*)dst = v;
        }
    }
}

}  // namespace gk
