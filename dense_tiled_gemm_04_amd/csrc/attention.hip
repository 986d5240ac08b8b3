// Attention forward (FlashAttention) on gfx950 for fp16 Q, K, V with fp32
// softmax state: the tutorial's fused attention kernel (news article on TileLang
// kernel design, paragraph on FlashAttention: query, key and value tiles, no
// attention matrix in global memory, an online softmax with running maxima,
// normalising sums and rescale factors, tiled matrix-core products, causal and
// non-causal; blog post on TileLang, "three-piece set" section, item 3).
//
//   O[i] = sum_j softmax_j(scale * Q[i] . K[j]) V[j],  j < Nkv (causal: j <= i)
//
// One workgroup = 4 wave64s owns a block of 128 query rows of one (batch, head);
// wave w owns rows 32w .. 32w+31 of it.  Per 64-key block:
//  * K and V tiles [64][D] sit in LDS, double-buffered; the next block's tiles
//    are copied by LDS-DMA (buffer_load_dwordx4 ... lds) while this block is
//    computed.  The buffer range check ends at key Nkv, so keys past the end
//    read as zeros (their scores are masked to -inf as well).
//  * Scores are computed transposed, S^T = K . Q^T, with
//    v_mfma_f32_32x32x16_f16: the A operand is K straight from LDS (ds_read_b128,
//    a key row is K-contiguous), the B operand is Q^T held in registers for the
//    whole loop.  In that layout lane l owns query row l % 32 and 16 keys per
//    32-key block, so the running max, the rescale factor and the running sum
//    of a row live in one lane (plus its partner lane l ^ 32).
//  * O^T += V^T . P^T with the same MFMA.  The B operand P^T needs, per lane,
//    8 keys of its query row; within every 16-key step the MFMA's k index is
//    mapped to keys so that these 8 are exactly 8 consecutive accumulator
//    registers of S^T (k = 8 (l/32) + 4 h + t  <->  key 8 h + 4 (l/32) + t).
//    P is converted to fp16 in place and needs no shuffle.  The A operand V^T
//    comes from two LDS transpose reads (ds_read_b64_tr_b16) per 16-key step,
//    using the same key mapping.
//  * The softmax state is fp32 and in the log2 domain: each probability is one
//    FMA (the scale folded in) and one v_exp_f32.  The reference maximum is
//    raised lazily, only when a row's maximum grows by more than 2^8, so the
//    accumulators are rarely rescaled and probabilities stay below 256.  A
//    block's probabilities are formed against the reference as it stands; the
//    block's maximum is formed only when some lane's sum of them reaches 2^8
//    (no probability can pass 2^8 while its lane's sum stays below).  The
//    probabilities enter the PV product rounded to fp16 in pairs, and the row
//    sum adds those same rounded values (v_dot2 with ones), so each output row
//    is an exact convex combination of value rows up to fp32 rounding.
//  * Key blocks that need no mask for any row of the workgroup run a loop body
//    without mask code; the boundary blocks run a second loop with it.
//  * Workgroup ids are remapped so that each XCD runs a contiguous range of
//    (batch, head, query block) tiles: a head's K and V are fetched into one L2.
//  * Causal: key blocks past the workgroup's last row are never visited; a wave
//    skips the blocks that lie wholly past its own rows; masks are applied only
//    in blocks that cross the diagonal or the end of the keys.  Workgroups are
//    launched longest-first.
// LDS tiles are XOR-swizzled in 16-byte chunks so that both read forms are free
// of bank conflicts.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attention_f16.h"
#include "common.h"
#include "gemm_f16.h"

using namespace gk;

namespace {

constexpr int FA_BM = 128;   // query rows per workgroup
constexpr int FA_BN = 64;    // keys per block
constexpr int FA_NW = 4;     // waves per workgroup
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLazyLog2 = 8.0f;  // rescale when a row maximum grows by more than 2^8
constexpr float kLazySum = 256.0f;  // 2^kLazyLog2

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct FaArgs {
    const f16* Q;
    const f16* K;
    const f16* V;
    f16* O;
    int Nq, Nkv;
    int q_blocks;
    float scale_log2;  // scale * log2(e)
};

// K tile [64][D]: logical chunk c of key row j at c ^ swz_k(j).  A ds_read_b128
// quarter-wave reads one logical chunk of 16 consecutive rows; the XOR puts
// them in 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int j) {
    return D == 128 ? (j & 15) : ((j >> 1) & 7);
}
// V tile [64][D]: a transpose read touches 4 consecutive rows x 64 bytes per
// half-wave; the XOR spreads those 16 chunks over distinct bank groups
// (D = 128: rows 256 bytes apart, shift by 4 chunks per row; D = 64: rows 128
// bytes apart, pairs of rows share a 256-byte window, shift every other pair).
template <int D>
__device__ __forceinline__ int swz_v(int j) {
    return D == 128 ? 4 * (j & 3) : 4 * ((j >> 1) & 1);
}

template <int D, bool CAUSAL, bool PRESCALE>
__global__ void __launch_bounds__(FA_NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
flash_attn_fwd_kernel(FaArgs p) {
    constexpr int CH = D / 8;                    // 16-byte chunks per row
    constexpr int TILE = FA_BN * D * 2;          // bytes of one K or V tile
    constexpr int INS = FA_BN * CH / (FA_NW * 64);  // copies per lane per tile
    constexpr int KS = D / 16;                   // k-steps of the score product
    constexpr int JB = FA_BN / 32;               // 32-key blocks per key block
    constexpr int DB = D / 32;                   // 32-column blocks of the output
    static_assert(D == 64 || D == 128, "head dimension");
    static_assert(INS * FA_NW * 64 == FA_BN * CH, "copy split");
    __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // K[2] | V[2]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int Nq = p.Nq, Nkv = p.Nkv;
    // Consecutive workgroup ids are dealt round-robin over the 8 XCDs; the remap
    // gives each XCD a contiguous run of ids, so the query blocks of one (batch,
    // head) share one L2 and fetch that head's K and V once per XCD.
    const int lid = xcd_contiguous_id((int)blockIdx.x, (int)gridDim.x);
    int qb = lid % p.q_blocks;
    const int64_t bh = lid / p.q_blocks;
    if (CAUSAL) qb = p.q_blocks - 1 - qb;  // longest rows first
    const int q0 = qb * FA_BM;
    const int row0 = q0 + 32 * wave_s;      // first query row of this wave
    const int i = row0 + (lane & 31);       // this lane's query row
    const f16* Qp = p.Q + bh * (int64_t)Nq * D;
    f16* Op = p.O + bh * (int64_t)Nq * D;

    // Q^T fragments for the whole loop: lane l holds Q[i][16 ks + 8 (l/32) .. +7].
    f16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (i < Nq) {
            qf[ks] = *(const f16x8*)(Qp + (int64_t)i * D + 16 * ks + 8 * (lane >> 5));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[ks][e] = (f16)0.0f;
        }
    }

    // copies: destination chunk P = (t * 4 + wave) * 64 + lane of a tile, key row P / CH
    const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.K + bh * (int64_t)Nkv * D), (short)0, Nkv * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.V + bh * (int64_t)Nkv * D), (short)0, Nkv * D * 2, 0x00020000);
    uint32_t k_off[INS], v_off[INS];
#pragma unroll
    for (int t = 0; t < INS; ++t) {
        const int P = (t * FA_NW + wave) * 64 + lane, jr = P / CH, pc = P % CH;
        k_off[t] = (uint32_t)((jr * D + 8 * (pc ^ swz_k<D>(jr))) * 2);
        v_off[t] = (uint32_t)((jr * D + 8 * (pc ^ swz_v<D>(jr))) * 2);
    }
    const uint32_t lds0 = lds_addr((GK_LDS char*)smem) + wave_s * 64 * 16;
    auto issue = [&](int jb, int buf) {
        const uint32_t kv = (uint32_t)jb * FA_BN * D * 2;
#pragma unroll
        for (int t = 0; t < INS; ++t) {
            dma_buffer_16(k_rsrc, k_off[t] + kv, lds0 + buf * TILE + t * FA_NW * 64 * 16);
            dma_buffer_16(v_rsrc, v_off[t] + kv, lds0 + (2 + buf) * TILE + t * FA_NW * 64 * 16);
        }
    };

    // LDS read offsets (bytes within a tile)
    int k_rd[JB][KS];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int jr = 32 * jj + (lane & 31), c = 2 * ks + (lane >> 5);
            k_rd[jj][ks] = jr * D * 2 + ((c ^ swz_k<D>(jr)) << 4);
        }
    // V^T: lane L = 16 g + 4 jq + q addresses V[key][col .. col+3] and receives
    // 4 keys of column 16 (g & 1) + L % 16; keys 16 step + 4 (g >> 1) + 8 h + jq.
    int v_rd[2][DB];
    {
        const int g = lane >> 4, jq = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int jr = 4 * (g >> 1) + 8 * h + jq, col = 32 * db + 16 * (g & 1) + 4 * q;
                v_rd[h][db] = jr * D * 2 + (((col >> 3) ^ swz_v<D>(jr)) << 4) + ((col & 7) << 1);
            }
    }
    // the V swizzle depends on the key row only through (j & 3) / ((j >> 1) & 1),
    // which a shift by a multiple of 16 keys keeps, so one offset per (h, db)
    // serves every 16-key step at + 16 step * D * 2 bytes.

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    // Softmax state of this lane's row, in the log2 domain: m_run is the
    // reference maximum (raised lazily, see below), l_run the sum of the fp16
    // probabilities applied so far (this lane's half of the keys).
    float m_run = -INFINITY, l_run = 0.0f;
    const float c = PRESCALE ? 1.0f : p.scale_log2;
    const f16x2 ones = {(f16)1.0f, (f16)1.0f};

    const int kv_blocks_all = (Nkv + FA_BN - 1) / FA_BN;
    const int kv_blocks = CAUSAL ? min(kv_blocks_all, (q0 + FA_BM - 1) / FA_BN + 1) : kv_blocks_all;
    // Blocks [0, n_plain) need no mask for any row of the workgroup: every key
    // exists and (causal) no key lies past the workgroup's first row.
    int n_plain = min(Nkv / FA_BN, kv_blocks);
    if (CAUSAL) n_plain = min(n_plain, (q0 + 1) / FA_BN);

    auto block = [&]<bool MASK>(int jb) {
        const int buf = jb & 1;
        wait_vmcnt0();
        __syncthreads();  // block jb in LDS for every wave; block jb-1's buffer free
        if (jb + 1 < kv_blocks) issue(jb + 1, buf ^ 1);
        const int kv0 = jb * FA_BN;
        if (CAUSAL && MASK && kv0 > row0 + 31) return;  // every key of the block is past this wave's rows

        const GK_LDS char* Ks = (const GK_LDS char*)smem + buf * TILE;
        const GK_LDS char* Vs = (const GK_LDS char*)smem + (2 + buf) * TILE;
        // S^T = K . Q^T; the two 32-key accumulators alternate so that no MFMA
        // waits for the one before it
        f32x16 sc[JB];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[jj][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
                const f16x8 kf = *(const GK_LDS f16x8*)(Ks + k_rd[jj][ks]);
                sc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], sc[jj], 0, 0, 0);
            }
        if constexpr (PRESCALE) {
#pragma unroll
            for (int jj = 0; jj < JB; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) sc[jj][r] *= p.scale_log2;
        }
        if constexpr (MASK) {
#pragma unroll
            for (int jj = 0; jj < JB; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = kv0 + 32 * jj + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (j >= Nkv || (CAUSAL && j > i)) sc[jj][r] = -INFINITY;
                }
        }
        // row maximum of the block in the log2 domain (raw maxima; c > 0), the lane and its partner l ^ 32
        auto block_max = [&]() {
            float mb = -INFINITY;
#pragma unroll
            for (int jj = 0; jj < JB; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) mb = fmaxf(mb, sc[jj][r]);
            return fmaxf(mb, __shfl_xor(mb, 32, 64)) * c;
        };
        // probabilities: exp2(s c - m) as one FMA and one v_exp_f32, rounded in
        // pairs to fp16 (v_cvt_pk_f16_f32) for the P^T operand; the block's sum
        // adds those same rounded pairs (v_dot2_f32_f16 with ones), so the
        // weights applied to V sum to one
        f16x8 pf[JB][2];
        auto probabilities = [&](float& l) {
#pragma unroll
            for (int jj = 0; jj < JB; ++jj)
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[jj][2 * k], c, -m_run));
                    const float b = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[jj][2 * k + 1], c, -m_run));
                    const f16x2 h = __builtin_convertvector((f32x2){a, b}, f16x2);
                    l = __builtin_amdgcn_fdot2(h, ones, l, false);
                    pf[jj][k >> 2][2 * (k & 3)] = h[0];
                    pf[jj][k >> 2][2 * (k & 3) + 1] = h[1];
                }
        };
        // Lazy rescaling: the reference maximum moves only when some row's block
        // maximum exceeds it by more than 2^8, so probabilities stay below 256
        // (exact enough in fp16, far from overflow) and the accumulators are
        // rescaled rarely.  The first block sets it from its own maximum (that
        // block holds key 0, which every row may see, so it is finite).  Later
        // blocks form their probabilities with the reference as it stands; each
        // is at most the sum of the block's probabilities the lane holds, so the
        // block's maximum is formed only when some lane's sum reaches 2^8.
        if (jb == 0) m_run = block_max();
        float l_blk = 0.0f;
        probabilities(l_blk);
        if (__any(l_blk >= kLazySum)) {
            const float mc = block_max();
            if (__any(mc > m_run + kLazyLog2)) {
                const float m_new = fmaxf(m_run, mc);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                l_blk = 0.0f;
                probabilities(l_blk);
            }
        }
        l_run += l_blk;
        // O^T += V^T . P^T, 16 keys per step
#pragma unroll
        for (int st = 0; st < FA_BN / 16; ++st) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const f16x4 v0 = lds_read_tr16_b64(Vs + v_rd[0][db] + st * 16 * D * 2);
                const f16x4 v1 = lds_read_tr16_b64(Vs + v_rd[1][db] + st * 16 * D * 2);
                const f16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[st >> 1][st & 1], oacc[db], 0, 0, 0);
            }
        }
    };

    if (kv_blocks > 0) issue(0, 0);
    int jb = 0;
    for (; jb < n_plain; ++jb) block.template operator()<false>(jb);
    for (; jb < kv_blocks; ++jb) block.template operator()<true>(jb);

    // normalise and write: lane l, register r of block db holds O[i][32 db + 8 (r/4) + 4 (l/32) + r % 4]
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.0f / l_tot;
    if (i < Nq) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f16x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = (f16)(oacc[db][4 * r4 + e] * inv);
                *(f16x4*)(Op + (int64_t)i * D + 32 * db + 8 * r4 + 4 * (lane >> 5)) = o;
            }
    }
}

// ---------------------------------------------------------------------------
// Software-pipelined forward kernel for D = 128 and 64.
//
// The block-serial kernel above runs, per 64-key block, the score MFMAs, then
// the softmax on the vector ALU, then the PV MFMAs; each stage waits for the
// one before, so a wave's matrix cores idle through its softmax.  A 32x32x16
// MFMA occupies the matrix core for 32 cycles, during which the same wave can
// issue independent vector instructions (about one exponential and two or three
// FMAs) at almost no cost.  This kernel therefore interleaves the stages of
// neighbouring blocks within each wave:
//   phase A(j): the score MFMAs of block j+1    || exponentials of block j, keys 32..63
//   phase B(j): the PV MFMAs of block j         || exponentials of block j+1, keys 0..31
// Each phase is a fixed sequence of 16 slots (8 at D = 64) fenced by scheduling
// barriers; a slot holds one MFMA, the LDS reads of a later slot's operand, and
// a share of the vector work (at D = 64 an exponential pair in every slot,
// at D = 128 in every other one).  A block's exponentials use the reference
// maximum as it stands.  The lazy-rescale test of the block-serial kernel (does the
// block's maximum exceed the reference by more than 2^8?) is taken between
// phases A(j) and B(j), once all of block j's probabilities exist, and without
// the block's maximum: each probability is at most the sum of those a lane
// holds, so a lane whose sum of the block's fp16 probabilities stays below 2^8
// holds none above 2^8.  Only when some lane's sum reaches 2^8 is the block's
// maximum formed; if it exceeds the reference by more than 2^8, the reference
// is raised, the accumulators and the running sum are rescaled and the block's
// probabilities are formed again.  The block-serial kernel takes the same test
// on the same probabilities; the two differ in the order of instructions and of
// the sums.  K and V tiles are copied one block apart: after the barrier that
// opens A(j), K(j+2) and V(j+1) are issued into the buffers that K(j) and
// V(j-1) have left, so two buffers of each suffice.
template <int D, bool CAUSAL, bool PRESCALE>
__global__ void __launch_bounds__(FA_NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
flash_attn_fwd_pipe_kernel(FaArgs p) {
    static_assert(D == 64 || D == 128, "head dimension");
    constexpr int CH = D / 8;
    constexpr int TILE = FA_BN * D * 2;
    constexpr int INS = FA_BN * CH / (FA_NW * 64);
    constexpr int KS = D / 16;   // k-steps of the score product (8 or 4)
    constexpr int DB = D / 32;   // output column blocks (4 or 2)
    constexpr int NSA = 2 * KS;  // MFMA slots of phase A (score MFMAs, two 32-key halves)
    constexpr int NSB = 4 * DB;  // MFMA slots of phase B (PV MFMAs, four 16-key steps)
    constexpr int EA = NSA / 8, EB = NSB / 8;  // slots per exponential pair (8 pairs per phase)
    constexpr int PDK = 3;       // K fragment reads issued this many slots ahead
    constexpr int PDV = 3;       // V fragment reads issued this many slots ahead
    static_assert(INS * FA_NW * 64 == FA_BN * CH, "copy split");
    __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // K[2] | V[2]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int Nq = p.Nq, Nkv = p.Nkv;
    const int lid = xcd_contiguous_id((int)blockIdx.x, (int)gridDim.x);
    int qb = lid % p.q_blocks;
    const int64_t bh = lid / p.q_blocks;
    if (CAUSAL) qb = p.q_blocks - 1 - qb;  // longest rows first
    const int q0 = qb * FA_BM;
    const int row0 = q0 + 32 * wave_s;
    const int i = row0 + (lane & 31);
    const f16* Qp = p.Q + bh * (int64_t)Nq * D;
    f16* Op = p.O + bh * (int64_t)Nq * D;

    f16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (i < Nq) {
            qf[ks] = *(const f16x8*)(Qp + (int64_t)i * D + 16 * ks + 8 * (lane >> 5));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[ks][e] = (f16)0.0f;
        }
    }

    const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.K + bh * (int64_t)Nkv * D), (short)0, Nkv * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.V + bh * (int64_t)Nkv * D), (short)0, Nkv * D * 2, 0x00020000);
    // Copy t of a tile moves the 4096 bytes after copy t - 1 (16 key rows at D = 128, 32 at D = 64); the
    // swizzle of a chunk depends on its row only through the row's low bits, which t does not change, so one
    // offset per lane serves every copy.
    uint32_t k_off0, v_off0;
    {
        const int jr = (wave * 64 + lane) / CH, pc = (wave * 64 + lane) % CH;
        k_off0 = (uint32_t)((jr * D + 8 * (pc ^ swz_k<D>(jr))) * 2);
        v_off0 = (uint32_t)((jr * D + 8 * (pc ^ swz_v<D>(jr))) * 2);
    }
    const uint32_t lds0 = lds_addr((GK_LDS char*)smem) + wave_s * 64 * 16;
    // Offsets derived from a base register are formed where they are used: an empty asm statement makes the
    // base opaque there, so that the compiler does not hoist the derived values out of the loop and hold
    // them in registers for its whole length.
    auto opaque = [](auto v) {
        asm volatile("" : "+v"(v));
        return v;
    };
    auto issue_k = [&](int jb) {
        const uint32_t kv = (uint32_t)jb * FA_BN * D * 2, ko = opaque(k_off0);
#pragma unroll
        for (int t = 0; t < INS; ++t)
            dma_buffer_16(k_rsrc, ko + (kv + t * 4096u), lds0 + (jb & 1) * TILE + t * FA_NW * 64 * 16);
    };
    auto issue_v = [&](int jb) {
        const uint32_t kv = (uint32_t)jb * FA_BN * D * 2, vo = opaque(v_off0);
#pragma unroll
        for (int t = 0; t < INS; ++t)
            dma_buffer_16(v_rsrc, vo + (kv + t * 4096u), lds0 + (2 + (jb & 1)) * TILE + t * FA_NW * 64 * 16);
    };

    // LDS read offsets.  K fragment of score slot s (k-step s/2, 32-key half s%2): key row 32 (s%2) + l%32,
    // 16-byte chunk (2 (s/2) + l/32) XOR swz_k(row); the swizzle depends on the row only through l%32, so the
    // row's high half and the k-step enter as 64 D (s%2) bytes and an XOR with 32 (s/2).  V^T fragment
    // (column block db, 8-key half h, 16-key step st) of the block-serial kernel: key row 4 (g/2) + 8 h + jq
    // + 16 st, columns 32 db + 16 (g%2) + 4 q; the swizzle depends on the row only through jq, so
    // 16 D h + 32 D st + (vbase XOR 64 db).
    const int kbase = ((lane & 31) * 2 * D) | (((lane >> 5) ^ swz_k<D>(lane & 31)) << 4);
    int vbase;
    {
        const int g = lane >> 4, jq = (lane >> 2) & 3, q = lane & 3;
        vbase = (4 * (g >> 1) + jq) * 2 * D + 16 * swz_v<D>(jq) + 32 * (g & 1) + 16 * (q >> 1) + 8 * (q & 1);
    }
    auto k_rd = [&](int kb, int s) { return 64 * D * (s & 1) + (kb ^ (32 * (s >> 1))); };
    auto v_rd = [&](int vb, int h, int db, int st) { return 16 * D * h + 32 * D * st + (vb ^ (64 * db)); };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    const f32x16 zero16 = {};
    float m_run, l_run = 0.0f, l_first = 0.0f;
    const float c = PRESCALE ? 1.0f : p.scale_log2;
    const f16x2 ones = {(f16)1.0f, (f16)1.0f};

    // scores of two blocks in flight (sc[parity][32-key half]) and their fp16 probabilities
    f32x16 sc[2][2];
    f16x8 pf[2][2][2];

    const int kv_blocks_all = (Nkv + FA_BN - 1) / FA_BN;
    const int n_wg = CAUSAL ? min(kv_blocks_all, (q0 + FA_BM - 1) / FA_BN + 1) : kv_blocks_all;
    const int n_w = CAUSAL ? min(kv_blocks_all, (row0 + 31) / FA_BN + 1) : kv_blocks_all;
    // blocks [0, n_plain) need no mask for any row of this wave
    int n_plain = min(Nkv / FA_BN, n_w);
    if (CAUSAL) n_plain = min(n_plain, (row0 + 1) / FA_BN);

    auto prepare = [&](f32x16 (&s)[2], int jb) {  // scale (non-positive scales) and mask one block's scores
        if constexpr (PRESCALE) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[jj][r] *= p.scale_log2;
        }
        if (jb >= n_plain) {
            const int kv0 = jb * FA_BN;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = kv0 + 32 * jj + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (j >= Nkv || (CAUSAL && j > i)) s[jj][r] = -INFINITY;
                }
        }
    };
    // partner lane l ^ 32 holds the other half of the row's keys
    auto row_max = [&](float m) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    };
    auto row_sum = [&](float v) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    };
    // probabilities of scores 2k, 2k+1 of one 32-key half, rounded to fp16 in a pair; the row sum adds the
    // same rounded values
    // The pair and the running sum pass through an empty asm statement, which keeps their computation in the
    // schedule slot where the pair is formed: the optimiser would otherwise sink this arithmetic to its
    // first use (past the end of the phase) and undo the interleaving with the MFMAs.
    auto exp_pair = [&](const f32x16& s, f16x8 (&pd)[2], int k, float m, float& l) {
        const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * k], c, -m));
        const float b = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * k + 1], c, -m));
        f16x2 h = __builtin_convertvector((f32x2){a, b}, f16x2);
        l = __builtin_amdgcn_fdot2(h, ones, l, false);
        asm volatile("" : "+v"(h), "+v"(l));
        pd[k >> 2][2 * (k & 3)] = h[0];
        pd[k >> 2][2 * (k & 3) + 1] = h[1];
    };
    auto max16 = [&](const f32x16& s, int h) {  // maximum of registers 8h .. 8h+7
        float m = fmaxf(s[8 * h], s[8 * h + 1]);
#pragma unroll
        for (int r = 2; r < 8; ++r) m = fmaxf(m, s[8 * h + r]);
        return m;
    };

    // ---- prologue: K(0), K(1), V(0) in LDS; block 0 scored, its reference maximum set, keys 0..31
    issue_k(0);
    if (n_wg > 1) issue_k(1);
    issue_v(0);
    wait_vmcnt0();
    __syncthreads();
    {
        const GK_LDS char* Ks = (const GK_LDS char*)smem;
        const int kb = opaque(kbase);
#pragma unroll
        for (int s = 0; s < 2 * KS; ++s) {
            const f16x8 kf = *(const GK_LDS f16x8*)(Ks + k_rd(kb, s));
            sc[0][s & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[s >> 1], s < 2 ? zero16 : sc[0][s & 1], 0, 0, 0);
        }
        prepare(sc[0], 0);
        const float mb = row_max(fmaxf(fmaxf(max16(sc[0][0], 0), max16(sc[0][0], 1)),
                                       fmaxf(max16(sc[0][1], 0), max16(sc[0][1], 1))));
        m_run = mb * c;  // the first block holds key 0, which every row may see: finite
#pragma unroll
        for (int k = 0; k < 8; ++k) exp_pair(sc[0][0], pf[0][0], k, m_run, l_first);
    }

    // The 8 exponential pairs of a phase go one per EA (EB) slots, on the last slot of each group.
    // phase A(j): score MFMAs of block j+1 (NEXT) || exponentials of block j, keys 32..63, summed into l_b
    auto phase_a = [&]<int PAR, bool NEXT>(float& l_b) {
        constexpr int NX = PAR ^ 1;
        const float mr = opaque(m_run);
        if constexpr (NEXT) {
            const GK_LDS char* Kn = (const GK_LDS char*)smem + NX * TILE;  // block j+1 has parity NX
            f16x8 kf[NSA];
            const int kb = opaque(kbase);
#pragma unroll
            for (int s = 0; s < PDK; ++s) kf[s] = *(const GK_LDS f16x8*)(Kn + k_rd(kb, s));
#pragma unroll
            for (int s = 0; s < NSA; ++s) {
                if (s + PDK < NSA) kf[s + PDK] = *(const GK_LDS f16x8*)(Kn + k_rd(kb, s + PDK));
                sc[NX][s & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[s], qf[s >> 1], s < 2 ? zero16 : sc[NX][s & 1],
                                                                        0, 0, 0);
                if (s % EA == EA - 1) exp_pair(sc[PAR][1], pf[PAR][1], s / EA, mr, l_b);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) exp_pair(sc[PAR][1], pf[PAR][1], k, mr, l_b);
        }
    };
    // phase B(j): PV MFMAs of block j || (NEXT) exponentials of block j+1, keys 0..31, formed with the reference
    // maximum as it stands and summed into l_half
    auto phase_b = [&]<int PAR, bool NEXT>(float& l_half) {
        constexpr int NX = PAR ^ 1;
        const GK_LDS char* Vs = (const GK_LDS char*)smem + (2 + PAR) * TILE;
        const float mr = opaque(m_run);
        f16x8 vf[NSB];
        const int vb = opaque(vbase);
        auto read_v = [&](int s) {
            const int st = s / DB, db = s % DB;
            const f16x4 v0 = lds_read_tr16_b64(Vs + v_rd(vb, 0, db, st));
            const f16x4 v1 = lds_read_tr16_b64(Vs + v_rd(vb, 1, db, st));
            vf[s] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
#pragma unroll
        for (int s = 0; s < PDV; ++s) read_v(s);
#pragma unroll
        for (int s = 0; s < NSB; ++s) {
            if (s + PDV < NSB) read_v(s + PDV);
            const int st = s / DB;
            oacc[s % DB] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[s], pf[PAR][st >> 1][st & 1], oacc[s % DB], 0, 0, 0);
            if constexpr (NEXT) {
                if (s % EB == EB - 1) exp_pair(sc[NX][0], pf[NX][0], s / EB, mr, l_half);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // The lazy-rescale test of block j (scores in sc[PAR]), whose probabilities are all formed: l0 and l1 are the
    // lane's sums of its first- and second-half probabilities.  A probability above 2^8 makes its lane's sum
    // reach 2^8; only then is the block's maximum formed and compared with the reference.  The sums then join
    // the running sum.
    auto settle = [&]<int PAR>(float l0, float l1) {
        if (__any(l0 + l1 >= kLazySum)) {
            const float mc = row_max(fmaxf(fmaxf(max16(sc[PAR][0], 0), max16(sc[PAR][0], 1)),
                                           fmaxf(max16(sc[PAR][1], 0), max16(sc[PAR][1], 1)))) * c;
            if (__any(mc > m_run + kLazyLog2)) {
                const float m_new = fmaxf(m_run, mc);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                l0 = 0.0f;
                l1 = 0.0f;
#pragma unroll
                for (int k = 0; k < 8; ++k) exp_pair(sc[PAR][0], pf[PAR][0], k, m_run, l0);
#pragma unroll
                for (int k = 0; k < 8; ++k) exp_pair(sc[PAR][1], pf[PAR][1], k, m_run, l1);
            }
        }
        l_run += l0 + l1;
    };

    // Each step opens with the barrier of block j and the copies of K(j+2) and V(j+1).  NEXT: block j+1 is
    // one of this wave's blocks (scored in phase A, its first half formed in phase B).  l_first carries the
    // first-half sum of the block a step forms next.
    auto open_step = [&](int j) {
        wait_vmcnt0();
        __syncthreads();  // K(j+1) and V(j) in LDS for every wave; K(j) and V(j-1) free
        if (j + 2 < n_wg) issue_k(j + 2);
        if (j + 1 < n_wg) issue_v(j + 1);
    };
    auto step = [&]<int PAR, bool NEXT>(int j) {
        constexpr int NX = PAR ^ 1;
        open_step(j);
        float l_second = 0.0f;
        phase_a.template operator()<PAR, NEXT>(l_second);
        settle.template operator()<PAR>(l_first, l_second);
        l_first = 0.0f;
        if constexpr (NEXT) prepare(sc[NX], j + 1);
        phase_b.template operator()<PAR, NEXT>(l_first);
    };

    // Blocks 0 .. n_w-1 are this wave's; the main loop runs only steps with a following block, so every
    // value it carries is written before it is read, and a tail of one or two steps closes the pipeline.
    // Waves whose causal rows end earlier then join the workgroup's remaining barriers and copies.
    int j = 0;
    for (; j + 2 < n_w; j += 2) {
        step.template operator()<0, true>(j);
        step.template operator()<1, true>(j + 1);
    }
    if (j + 1 < n_w) {
        step.template operator()<0, true>(j);
        step.template operator()<1, false>(j + 1);
        j += 2;
    } else {
        step.template operator()<0, false>(j);
        j += 1;
    }
    for (; j < n_wg; ++j) open_step(j);

    const float inv = 1.0f / row_sum(l_run);
    if (i < Nq) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f16x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = (f16)(oacc[db][4 * r4 + e] * inv);
                *(f16x4*)(Op + (int64_t)i * D + 32 * db + 8 * r4 + 4 * (lane >> 5)) = o;
            }
    }
}

template <int D, bool CAUSAL, bool PRESCALE>
hipError_t launch(const FaArgs& a, int64_t BH, hipStream_t s) {
    hipLaunchKernelGGL((flash_attn_fwd_kernel<D, CAUSAL, PRESCALE>), dim3((unsigned)(BH * a.q_blocks)),
                       dim3(FA_NW * 64), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FaArgs& a, int64_t BH, bool causal, bool prescale, hipStream_t s) {
    if (prescale) return causal ? launch<D, true, true>(a, BH, s) : launch<D, false, true>(a, BH, s);
    return causal ? launch<D, true, false>(a, BH, s) : launch<D, false, false>(a, BH, s);
}

template <int D, bool CAUSAL, bool PRESCALE>
hipError_t launch_pipe(const FaArgs& a, int64_t BH, hipStream_t s) {
    hipLaunchKernelGGL((flash_attn_fwd_pipe_kernel<D, CAUSAL, PRESCALE>), dim3((unsigned)(BH * a.q_blocks)),
                       dim3(FA_NW * 64), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_pipe_d(const FaArgs& a, int64_t BH, bool causal, bool prescale, hipStream_t s) {
    if (prescale) return causal ? launch_pipe<D, true, true>(a, BH, s) : launch_pipe<D, false, true>(a, BH, s);
    return causal ? launch_pipe<D, true, false>(a, BH, s) : launch_pipe<D, false, false>(a, BH, s);
}

}  // namespace

extern "C" {

int flash_attn_fwd_f16(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D, const void* Q, const void* K,
                       const void* V, void* O, int causal, float scale, void* stream) {
    return flash_attn_fwd_f16_kernel(B, H, Nq, Nkv, D, Q, K, V, O, causal, scale, FLASH_ATTN_KERNEL_AUTO, stream);
}

int flash_attn_fwd_f16_kernel(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D, const void* Q,
                              const void* K, const void* V, void* O, int causal, float scale, int kernel,
                              void* stream) {
    if (kernel != FLASH_ATTN_KERNEL_AUTO && kernel != FLASH_ATTN_KERNEL_BLOCK_SERIAL &&
        kernel != FLASH_ATTN_KERNEL_PIPELINED)
        return GEMM_ERR_NO_CONFIG;
    if (B < 0 || H < 0 || Nq < 0 || Nkv < 0 || D < 0) return GEMM_ERR_INVALID_DIM;
    if (B == 0 || H == 0 || Nq == 0) return GEMM_OK;
    if (Nkv == 0) return GEMM_ERR_INVALID_DIM;  // a query with no key has no softmax
    if (D != 64 && D != 128) return GEMM_ERR_UNSUPPORTED;
    if (!isfinite(scale) || fabsf(scale) > 1e30f) return GEMM_ERR_INVALID_DIM;
    if (!Q || !K || !V || !O) return GEMM_ERR_NULL_POINTER;
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) % 16 != 0) return GEMM_ERR_MISALIGNED;
    const int64_t q_blocks = (Nq + FA_BM - 1) / FA_BM;
    // 32-bit buffer sizes per (batch, head) slab and a 32-bit grid
    if (Nkv * D * 2 > INT32_MAX - 1024 || Nq > INT32_MAX / 2 || B * H * q_blocks > INT32_MAX)
        return GEMM_ERR_INVALID_DIM;
    FaArgs a;
    a.Q = (const f16*)Q;
    a.K = (const f16*)K;
    a.V = (const f16*)V;
    a.O = (f16*)O;
    a.Nq = (int)Nq;
    a.Nkv = (int)Nkv;
    a.q_blocks = (int)q_blocks;
    a.scale_log2 = scale * kLog2e;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    // a positive scale is folded into the exponent's FMA (the row maximum of the
    // raw scores is the maximum of the scaled ones); otherwise scores are
    // scaled first
    const bool prescale = !(scale > 0.0f);
    if (kernel != FLASH_ATTN_KERNEL_BLOCK_SERIAL)
        e = D == 128 ? launch_pipe_d<128>(a, B * H, causal != 0, prescale, s)
                     : launch_pipe_d<64>(a, B * H, causal != 0, prescale, s);
    else
        e = D == 128 ? launch_d<128>(a, B * H, causal != 0, prescale, s)
                     : launch_d<64>(a, B * H, causal != 0, prescale, s);
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // extern "C"
