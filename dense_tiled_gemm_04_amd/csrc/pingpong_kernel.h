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
// group per SIMD (waves w and w + 4 share a SIMD): group 0 owns rows 0-127 of
// the 256x256 tile, group 1 rows 128-255, and wave wn of a group the 64
// columns 64 wn .. 64 wn + 63, i.e. a 128x64 sub-tile of 8x4
// v_mfma_f32_16x16x32_f16 blocks with its 128 fp32 accumulators pinned to
// AGPRs.  Time runs in phases separated by workgroup barriers; in every phase
// one group computes and the other loads:
//   computing: the 64 MFMAs of one 64-deep stage (two k-steps of 32), back to
//              back, from fragments already in registers;
//   loading:   the LDS reads of its next stage's fragments (16 A reads and 16
//              B transpose reads, or 8 B reads with B transposed), its share
//              of the global -> LDS copies, and a wait for the reads.
// Group 0 loads stage u in phase 2u and computes it in phase 2u + 1; group 1
// does both one phase later.  On each SIMD one wave keeps the matrix core
// busy while its partner reads LDS and issues copies; memory instructions of
// the partner leave the MFMA wave's issue rate intact (measured on this part:
// 16-17 cycles per 16x16x32 MFMA with the partner idle, reading LDS or
// copying), which is what makes the split pay.  A 64-deep stage gives each
// phase ~1,100 MFMA cycles against the loads' latency.
//
// LDS holds two stages, each the A tile [256][64] and the B tile [64][256]
// (Bt: [256][64]), 64 KiB per stage, 128 KiB in all.  Stage u lives in slot
// u mod 2; group 0 reads it in phase 2u, group 1 in phase 2u + 1, each waiting
// for its reads before the barrier that ends its phase.  Copies of stage u + 2
// go into the same slot once both groups have read stage u:
//   B's by group 1 at the end of phase 2u + 1, after its own reads of stage u
//   have completed; it waits for them two phases later (before group 0 reads
//   stage u + 2 in phase 2u + 4);
//   A's by group 0 in phase 2u + 2 (its load phase of stage u + 1); it waits
//   for them at the end of its next compute phase.
// Copy layout, swizzles and the epilogue are those of gemm_tile_pipe_kernel
// with a 64-deep K block: XOR-swizzled 16-byte chunks (bank-conflict-free
// ds_read_b128 and ds_read_b64_tr_b16), and the C tile staged through the
// freed slots and written with row-contiguous 16-byte stores (non-temporal
// with NT).  Requires whole tiles: M % 256 == 0, N % 256 == 0, K % 64 == 0,
// 16-byte-aligned rows of A, B and C and an 8-byte-aligned bias.
#pragma once
#include "common.h"
#include "tile_pipe_kernel.h"

namespace gk {

constexpr int PP_BM = 256, PP_BN = 256, PP_BK = 64, PP_SLOTS = 2, PP_WAVES = 8;
constexpr int PP_SLOT_A = PP_BM * PP_BK * 2;   // 32 KiB
constexpr int PP_SLOT_B = PP_BK * PP_BN * 2;   // 32 KiB
constexpr int PP_LDS_BYTES = PP_SLOTS * (PP_SLOT_A + PP_SLOT_B);

template <int GROUP_M, int EPI, int BT, int NT_C>
__global__ void __launch_bounds__(PP_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_pingpong_kernel(GemmArgs p) {
    constexpr int BM = PP_BM, BN = PP_BN, BK = PP_BK, MF = 16, KS = BK / 32;  // two k-steps of 32 per stage
    constexpr int WTM = 128, WTN = 64, TM = WTM / MF, TN = WTN / MF;          // 8 x 4 MFMA blocks per wave
    constexpr int CA = BK / 8, CB = BN / 8;                                    // 16-byte chunks per row
    constexpr int NCOPY = 8;                                                   // copies per lane per stage
    static_assert(PP_LDS_BYTES <= 160 * 1024 && BM * BN * 2 <= PP_LDS_BYTES, "LDS budget; C tile fits the slots");
    static_assert(BM * CA == NCOPY * 4 * 64 && (BT ? BN * CA : BK * CB) == NCOPY * 4 * 64, "one group copies an operand");
    static_assert(TN == 4 && TM % 2 == 0 && KS == 2, "the MFMA blocks are written for 4 column blocks and pairs of rows");

    __shared__ __attribute__((aligned(1024))) char smem_raw[PP_LDS_BYTES];
    GK_LDS char* const a_lds = (GK_LDS char*)smem_raw;                 // [SLOTS][BM][BK]
    GK_LDS char* const b_lds = a_lds + PP_SLOTS * PP_SLOT_A;           // [SLOTS][BK][BN] (Bt: [SLOTS][BN][BK])

    const int K = p.K, lda = p.lda, ldb = p.ldb, ldc = p.ldc;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);          // 0: rows 0-127, 1: rows 128-255
    const int wl = __builtin_amdgcn_readfirstlane(wave & 3);            // wave within the group
    int tm, tn;
    {
        const int nwg = p.tiles_m * p.tiles_n;
        grouped_tile<GROUP_M>(xcd_contiguous_id((int)blockIdx.x, nwg), p.tiles_m, p.tiles_n, tm, tn);
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int KT = K / BK;  // stages (K % 64 == 0, host-checked)

    // Fragment read offsets (bytes within a slot).  A: k-step ks, row block mi at a_rd[ks] + mi * 16 rows
    // (the swizzle depends on a row through (row / 2) % 8, which 16 rows do not change).
    int a_rd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int row = grp * WTM + (lane % MF);
        a_rd[ks] = row * BK * 2 + (((4 * ks + lane / MF) ^ swz_a<BK>(row)) << 4);
    }
    // B: transpose reads of k-rows 32 ks + 8 (l/16) + 4 h + (l/4) % 4 at b_rd[ni] + (32 ks + 4 h) k-rows (the
    // swizzle depends on a k-row through bits 0, 1 and 3, which 4 h and 32 ks do not change).  Bt: rows of the
    // [BN][BK] tile like A's.
    int b_rd[BT ? 1 : TN];
    int bt_rd[BT ? KS : 1];
    if constexpr (!BT) {
        const int g4 = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
        const int kr = 8 * g4 + j;
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            const int nl = wl * WTN + ni * MF + 4 * q;
            b_rd[ni] = kr * BN * 2 + (((nl >> 3) ^ swz_b<BN, MF>(kr)) << 4) + ((nl & 7) << 1);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int row = wl * WTN + (lane % MF);
            bt_rd[ks] = row * BK * 2 + (((4 * ks + lane / MF) ^ swz_a<BK>(row)) << 4);
        }
    }

    // Copy sources.  Group 0 copies A, group 1 copies B (or Bt).  Copy j of wave wl fills destination chunk
    // P = (4 j + wl) * 64 + lane of the stage's tile, whose source is the logical chunk the swizzle puts there.
    //   A and Bt ([256][64], 8 chunks per row): row (4 j + wl) * 8 + l/8, i.e. 32 rows per j, and the row's
    //   swizzle ((row / 2) % 8) is the same for every j: source c_off[0] + j * 32 rows.
    //   B ([64][256], 32 chunks per k-row): k-row (4 j + wl) * 2 + l/32, i.e. 8 k-rows per j; the swizzle
    //   depends on bit 3 of the k-row, so on j's parity: source c_off[j % 2] + (j / 2) * 16 k-rows.
    const bool rows_of_a = grp == 0 || BT;  // this group's operand is stored [256][64]
    uint32_t c_off[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int P = (par * 4 + wl) * 64 + lane;
        if (rows_of_a) {
            const int r = P / CA, c = (P % CA) ^ swz_a<BK>(r);
            c_off[par] = (uint32_t)((r * (grp == 0 ? lda : ldb) + 8 * c) * 2);
        } else {
            const int kr = P / CB, c = (P % CB) ^ swz_b<BN, MF>(kr);
            c_off[par] = (uint32_t)((kr * ldb + 8 * c) * 2);
        }
    }
    const size_t row_step = rows_of_a ? (size_t)32 * (grp == 0 ? lda : ldb) * 2 : (size_t)16 * ldb * 2;
    const char* const a_row0 = (const char*)(p.A + (size_t)m0 * lda);
    const char* const b_col0 = (const char*)(BT ? p.B + (size_t)n0 * ldb : p.B + n0);
    const uint32_t lds_dst0 = (grp == 0 ? lds_addr(a_lds) : lds_addr(b_lds)) + wl * 64 * 16;
    const int slot_bytes = grp == 0 ? PP_SLOT_A : PP_SLOT_B;
    // The copy source is a scalar operand of the inline-asm copy.  The tile origin comes out of the tile-order
    // arithmetic in vector registers, so this group's operand origin passes through readfirstlane here, once
    // (it is the same in every lane), and every copy address is derived from it by scalar arithmetic.  A
    // readfirstlane placed next to a copy would break a rule the compiler enforces for its own memory
    // instructions but not inside inline asm: an SGPR written by a VALU instruction may be read as a memory
    // address only 5 wait states later, else the load sees the register's previous contents.
    const char* const op0 = [&] {
        const uint64_t v = (uint64_t)(uintptr_t)(grp == 0 ? a_row0 : b_col0);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
        return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
    }();
    const size_t stage_step = rows_of_a ? (size_t)BK * 2 : (size_t)BK * ldb * 2;  // bytes between stages
    // this wave's copies of stage v into slot v mod 2
    auto copy = [&](int v) {
        const char* src = op0 + (size_t)v * stage_step;
        const uint32_t dst = lds_dst0 + (v & (PP_SLOTS - 1)) * slot_bytes;
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) {
            const char* s = src + (rows_of_a ? (size_t)j * row_step : (size_t)(j >> 1) * row_step);
            dma_global_16(s, rows_of_a ? c_off[0] : c_off[j & 1], dst + j * 4 * 64 * 16);
        }
    };

    constexpr int NACC = 4;
    typedef float accv __attribute__((ext_vector_type(NACC)));
    accv acc[TM][TN];
#pragma unroll
    for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) acc[mi][ni] = accv{0.f, 0.f, 0.f, 0.f};
    f16x8 fa[KS][TM];
    f16x4 fb[BT ? 1 : KS][BT ? 1 : TN][2];
    f16x8 fbt[BT ? KS : 1][BT ? TN : 1];

    auto load_frags = [&](int u) {
        const int s = u & (PP_SLOTS - 1);
        const GK_LDS char* As = a_lds + s * PP_SLOT_A;
        const GK_LDS char* Bs = b_lds + s * PP_SLOT_B;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int ni = 0; ni < TN; ++ni) {
                if constexpr (BT) {
                    fbt[ks][ni] = *(const GK_LDS f16x8*)(Bs + bt_rd[ks] + ni * MF * BK * 2);
                } else {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        fb[ks][ni][h] = lds_read_tr16_b64(Bs + b_rd[ni] + (32 * ks + 4 * h) * BN * 2);
                }
            }
#pragma unroll
            for (int mi = 0; mi < TM; ++mi) fa[ks][mi] = *(const GK_LDS f16x8*)(As + a_rd[ks] + mi * MF * BK * 2);
        }
    };
    // The 64 MFMAs of a stage, issued only when `go` is nonzero.  The test and the branch sit inside the asm
    // blocks, so to the compiler the accumulators are updated in place on every path: a branch around them in
    // the source would join two versions of all 128 accumulators, which the register allocator copies and
    // spills.  Each block takes two A rows of one k-step (8 MFMAs).
    auto mfma_all = [&](int go) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            f16x8 b[TN];
#pragma unroll
            for (int ni = 0; ni < TN; ++ni) {
                if constexpr (BT) {
                    b[ni] = fbt[ks][ni];
                } else {
                    b[ni] = __builtin_shufflevector(fb[ks][ni][0], fb[ks][ni][1], 0, 1, 2, 3, 4, 5, 6, 7);
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
                    : [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]), [a0] "v"(fa[ks][mp]),
                      [a1] "v"(fa[ks][mp + 1]), [go] "s"(go)
                    : "scc");
            }
        }
    };
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

    // Prologue: stages 0 and 1 copied (each group its operand) and landed everywhere before phase 0.
    copy(0);
    if (KT > 1) copy(1);
    wait_vmcnt0();
    __syncthreads();

    // Phases t = 0 .. 2 KT, one barrier after each.  In phase t a wave of group g is s = t - g phases into its
    // own sequence: s even loads stage s/2, s odd computes stage (s-1)/2.  One code path serves both groups,
    // so the accumulators and fragments have a single home in registers.
    for (int t = 0; t <= 2 * KT; ++t) {
        const int st = t - grp;
        const bool loading = st >= 0 && (st & 1) == 0 && (st >> 1) < KT;
        const int computing = st >= 0 && (st & 1) == 1;  // stage (st - 1) / 2 < KT, as st <= 2 KT - grp
        if (loading) {
            const int u = st >> 1;
            // group 0: A of stage u + 1 into the slot that stage u - 1 has left (stages 0 and 1: prologue)
            if (grp == 0 && u >= 1 && u + 1 < KT) copy(u + 1);
            load_frags(u);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (grp == 1) {
                // B of stage u + 2 into this slot, now that both groups have read stage u; then B of stage u + 1
                // (issued two phases ago) must have landed before group 0 reads it in the next phase
                if (u + 2 < KT) {
                    copy(u + 2);
                    wait_vmcnt<NCOPY>();
                } else {
                    wait_vmcnt0();
                }
            }
        }
        mfma_all(__builtin_amdgcn_readfirstlane(computing));
        if (grp == 0 && computing) wait_vmcnt0();  // A of stage u + 1 landed before group 0 reads it
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
    __syncthreads();  // every wave has finished reading the slots
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
        const int nc = ni * MF + 4 * (lane_e >> 4);
        const int n = n0 + wn_e * WTN + nc;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (EPI != EPI_NONE) {
            const f16x4 b4 = *(const f16x4*)(p.bias + n);  // whole tiles: n + 4 <= N
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[e] = (float)b4[e];
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
        f16* dst = p.C + (size_t)m * ldc + n;
        if constexpr (NT_C) {
            __builtin_nontemporal_store(v, (f16x8*)dst);
        } else {
            *(f16x8*)dst = v;
        }
    }
}

}  // namespace gk
