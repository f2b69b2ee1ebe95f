// gemm_f8.hpp -- GEMM on 8-bit floating-point operands (E4M3 or E5M2, each
// operand its own format) with fp32 accumulation, for gfx950.
//
// C = A * B^T, A stored M x K and B stored N x K (both K-contiguous: the
// Croqtile tutorial ch.4 form with the [N,K] right operand), with the scales
// of the same chapter's FP8 variant: the contraction of each operand pair is
// multiplied by the two operands' scales after it is formed, inside the
// kernel, with no separate dequantisation pass.  Two kinds of scale, both
// optional:
//   * block scales: one E8M0 byte (2^(e - 127)) per row of A (and of B) and
//     per 32-element block of K.  They are the scale operands of
//     v_mfma_scale_f32_32x32x64_f8f6f4 itself, so a block's contraction and
//     its scaling are one instruction (the fused form).
//   * row scales: one fp32 value per row of A and per row of B (or one per
//     operand), applied to the finished fp32 sums in the epilogue (the
//     separate scale statement).
//
// The structure is that of the 16-bit direct-load kernel: one workgroup per
// output tile, the K loop inside the workgroup, direct global -> LDS loads
// of 16-byte granules into a K-contiguous, XOR-swizzled LDS layout; a K
// tile is 128 bytes of each row (128 elements), i.e. the same 8 granules per
// row as a 64-element 16-bit tile, so the LDS geometry, the swizzle and the
// load addressing carry over with bytes for elements.
//
// MFMA operand layout (32 x 32 x 64, measured on gfx950): lane l supplies
// row l % 32 of its operand; its 32 bytes are two 16-byte halves, bytes
// 0..15 holding k = 16 g .. 16 g + 15 and bytes 16..31 holding k = 32 + 16 g
// .. 32 + 16 g + 15 (g = l / 32).  The scale operand of lane l (the byte
// chosen by op_sel) scales K block 0 (k 0..31) of row l when l < 32 and K
// block 1 (k 32..63) of row l - 32 otherwise.  Result: lane l, register r
// holds D[8 (r / 4) + 4 g + r % 4][l % 32].  With B as the first operand,
// lane l ends with C[m = l % 32][n = 8 (r / 4) + 4 g + r % 4]: four runs of
// four consecutive output columns.
//
// K step ks (0, 1) of a K tile covers k = 64 ks .. 64 ks + 63: lane l reads
// granules 4 ks + g and 4 ks + 2 + g of its row, and its scale must be the
// one of block 4 kt + 2 ks + g of the whole K range.  The four block-scale
// bytes of a row for K tile kt are dword kt % 4 of the row's 16 bytes for
// K tiles 4h .. 4h + 3 (h = kt / 4); those 16 bytes of every row of the
// workgroup's A and B tiles travel to LDS together (one direct 16-byte load
// per row, with the data of K tile 4h) into one of two group buffers.  At
// the start of K tile kt each lane reads its dwords for the tile and packs
// two fragments' bytes into one register with one byte permute: bytes
// (g, 2 + g) of fragment 2p at positions (0, 2), those of fragment 2p + 1
// at (1, 3); op_sel = 2 ks + (fragment % 2) then picks the scale.
#pragma once

#include "gemm_m16.hpp"

namespace tdg {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// One scaled 32 x 32 x 64 MFMA: first operand x of format FX with scale byte
// OPX of sx, second operand y of format FY with scale byte OPY of sy
// (formats: 0 = E4M3, 1 = E5M2).
template <int FX, int FY, int OPX, int OPY>
__device__ __forceinline__ f32x16 mfma_f8(u32x4 xl, u32x4 xh, u32x4 yl, u32x4 yh, f32x16 c, int sx, int sy) {
    const i32x8 x = __builtin_bit_cast(i32x8, __builtin_shufflevector(xl, xh, 0, 1, 2, 3, 4, 5, 6, 7));
    const i32x8 y = __builtin_bit_cast(i32x8, __builtin_shufflevector(yl, yh, 0, 1, 2, 3, 4, 5, 6, 7));
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, FX, FY, OPX, sx, OPY, sy);
}

// dma16 issued only when `issue` (wave-uniform) is nonzero.  The test and
// the skip are inside the assembly, so the kernel's code around it stays one
// basic block and the compiler's instruction schedule is not split there.
template <uint32_t IMM>
__device__ __forceinline__ void dma16_if(u32x4 rsrc, uint32_t voff, uint32_t lds_base, uint32_t issue) {
    uint32_t saved;
    asm volatile(
        "s_cmp_eq_u32 %5, 0\n\t"
        "s_cbranch_scc1 1f\n\t"
        "s_mov_b32 %0, m0\n\t"
        "s_add_u32 m0, %3, %4\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0\n"
        "1:"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"(lds_base), "n"(IMM), "s"(issue)
        : "memory", "scc");
}

// Record count of `bytes` valid bytes (clamped to [0, 2^31 - 1]).
__device__ __forceinline__ uint32_t records_bytes(int64_t bytes) {
    return bytes <= 0 ? 0u : (bytes >= (int64_t)BUF_RECORDS ? (uint32_t)BUF_RECORDS : (uint32_t)bytes);
}

// BM x BN workgroup tile, WM x WN waves of (BM/WM) x (BN/WN), K tiles of
// 128 in STAGES LDS stages.  FA, FB: formats of A and B.  BSCALE: whether
// block scales are applied (without them the MFMA scale operands are 1).
template <int BM, int BN, int WM, int WN, int STAGES, int FA, int FB, bool BSCALE, int CT>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f8_kernel(F8Args p) {
    constexpr int BK = 128, KG = 8;
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int RM = WTM / 32, RN = WTN / 32;
    static_assert(RM * 32 == WTM && RN * 32 == WTN, "wave tile must be a multiple of 32");
    static_assert(RM % 2 == 0 && RN % 2 == 0, "fragments pair up for the packed scales");
    static_assert(NW % 2 == 0, "an even number of waves");
    constexpr int A_SLOTS = BM * KG, B_SLOTS = BN * KG;
    constexpr int STAGE = A_SLOTS + B_SLOTS;
    constexpr int SG = BSCALE ? BM + BN : 0;        // slots of one scale group buffer (16 bytes per row)
    constexpr int NIA = A_SLOTS / 64, NIB = B_SLOTS / 64, NIS = BSCALE ? (BM + BN) / 64 : 0;
    static_assert(NIA % NW == 0 && NIB % NW == 0 && NIS % NW == 0, "whole load instructions per wave");
    constexpr int QA = NIA / NW, QB = NIB / NW, QS = NIS / NW, NDMA = QA + QB;
    static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 stages");
    static_assert((STAGES - 1) * NDMA + 1 < 64, "vmcnt range");
    static_assert((STAGE * STAGES + 2 * SG) * 16 <= 160 * 1024, "LDS budget");
    constexpr uint32_t SOFF = (uint32_t)(STAGE * STAGES) * 16u;   // byte offset of the scale group buffers

    __shared__ u32x4 smem[STAGES * STAGE + 2 * SG];

    int batch, tm, tn;
    tile_of(p, xcd_order(blockIdx.x, gridDim.x), batch, tm, tn);
    (void)batch;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave / WN, wave_n = wave % WN;
    const int M = p.M, N = p.N, K = p.K;
    const int nk = (K + BK - 1) / BK;
    const int nkb = (K + 31) / 32;                  // 32-element K blocks
    const int m0 = tm * BM, n0 = tn * BN;
    const int64_t lda = p.lda, ldb = p.ldb;
    const uint8_t *Atile = p.A + (int64_t)m0 * lda;
    const uint8_t *Btile = p.B + (int64_t)n0 * ldb;
    const int a_rows = M - m0 < BM ? M - m0 : BM;
    const int b_rows = N - n0 < BN ? N - n0 : BN;

    // ---- direct-load addressing (the 16-bit kernel's K-contiguous layout) ----
    // Load q of this wave is instruction t = q*NW + wave: rows 8t .. 8t+7,
    // 8 granules each; the lane's row is 8t + lane/8, its granule
    // (lane%8) ^ kx16(row), and kx16 does not depend on q (NW is even).
    const int kc_row = wave * 8 + (lane >> 3);
    const int kc_g = (lane & 7) ^ kx16(kc_row);
    const int kc_klim = K - kc_g * 16;              // granule loaded while k0 < kc_klim
    const uint32_t a_lane = (uint32_t)(kc_row * lda + kc_g * 16);
    const uint32_t a_qs = (uint32_t)(NW * 8 * lda);
    const uint32_t b_lane = (uint32_t)(kc_row * ldb + kc_g * 16);
    const uint32_t b_qs = (uint32_t)(NW * 8 * ldb);
    // Scale load q of this wave is instruction t = q*NW + wave over the rows
    // of A (t < BM/64) then of B: lane l fetches the 16 scale bytes of K
    // tiles 4h .. 4h + 3 of row 64 t' + l, which land in group buffer h % 2
    // at 16 * (row index in the tile list).
    const uint8_t *s_base[QS > 0 ? QS : 1];
    uint32_t s_off[QS > 0 ? QS : 1];
#pragma unroll
    for (int q = 0; q < QS; ++q) {
        const int t = q * NW + wave;
        // (an operand without block scales loads nothing: every offset is
        // out of range, and its scale operands are set to 1 below)
        if (t < BM / 64) {
            const int r = 64 * t + lane;
            s_base[q] = p.xa + (int64_t)m0 * p.ldxa;
            s_off[q] = (p.xa != nullptr && r < a_rows) ? (uint32_t)(r * p.ldxa) : OOB_OFFSET;
        } else {
            const int r = 64 * (t - BM / 64) + lane;
            s_base[q] = p.xb + (int64_t)n0 * p.ldxb;
            s_off[q] = (p.xb != nullptr && r < b_rows) ? (uint32_t)(r * p.ldxb) : OOB_OFFSET;
        }
    }

    auto dma_op = [&](auto qtag, int kt, u32x4 *st) {
        constexpr int q = decltype(qtag)::value;
        const int k0 = kt * BK;
        if constexpr (q < QA) {
            const uint32_t base = lds_addr_of(st) + (uint32_t)wave * 1024u;
            const u32x4 rs = rsrc_words_n(Atile + k0, records_bytes((int64_t)(a_rows - 1) * lda + K - k0));
            const uint32_t off = (k0 < kc_klim ? a_lane : OOB_OFFSET) + (uint32_t)q * a_qs;
            dma16<(uint32_t)(q * NW) * 1024u>(rs, off, base);
        } else if constexpr (q < QA + QB) {
            constexpr int qb = q - QA;
            const uint32_t base = lds_addr_of(st) + (uint32_t)wave * 1024u;
            const u32x4 rs = rsrc_words_n(Btile + k0, records_bytes((int64_t)(b_rows - 1) * ldb + K - k0));
            const uint32_t off = (k0 < kc_klim ? b_lane : OOB_OFFSET) + (uint32_t)qb * b_qs;
            dma16<(uint32_t)(A_SLOTS * 16 + qb * NW * 1024)>(rs, off, base);
        }
    };
    // With the data of K tile kt, when kt starts a group of four (and is a
    // tile of the product), the scale group of K tiles kt .. kt + 3, issued
    // first so that the waits for tile kt cover it too.
    auto scale_group = [&](int kt) {
        if constexpr (BSCALE) {
            const int h = kt >> 2;
            const uint32_t issue = __builtin_amdgcn_readfirstlane((uint32_t)(((kt & 3) == 0) & (kt < nk)));
            const uint32_t base = lds_addr_of(smem) + SOFF + (uint32_t)(h & 1) * (SG * 16u) + (uint32_t)wave * 1024u;
            static_for<0, QS>([&](auto qtag) {
                constexpr int qs = decltype(qtag)::value;
                const u32x4 rs = rsrc_words(s_base[qs] + 16 * h);
                dma16_if<(uint32_t)(qs * NW) * 1024u>(rs, s_off[qs], base, issue);
            });
        }
    };
    auto issue_to = [&](int kt, u32x4 *st) {
        scale_group(kt);
        static_for<0, NDMA>([&](auto q) { dma_op(q, kt, st); });
    };

    // ---- fragment addresses ----
    // A fragment i, half h at K step ks: row wave_m*WTM + 32 i + lane%32,
    // granule 4 ks + 2 h + lane/32; kx16 of that row is (lane>>1)&7 for
    // every i.  B alike.
    const int fr = lane & 31, fg = lane >> 5;
    int a_b[2][2], b_b[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            a_b[ks][h] = (wave_m * WTM + fr) * KG + ((4 * ks + 2 * h + fg) ^ ((fr >> 1) & 7));
            b_b[ks][h] = (wave_n * WTN + fr) * KG + ((4 * ks + 2 * h + fg) ^ ((fr >> 1) & 7));
        }
    const int sa_w = 4 * (wave_m * WTM + fr);              // scale dwords of A fragment 0's row
    const int sb_w = 4 * (BM + wave_n * WTN + fr);         // ... of B fragment 0's row
    // the scale dwords of K tile kt: group buffer (kt / 4) % 2, dword kt % 4
    auto scale_ptr = [&](int kt) {
        return reinterpret_cast<const uint32_t *>(smem + STAGE * STAGES + ((kt >> 2) & 1) * SG) + (kt & 3);
    };

    constexpr int NFR = 2 * (RM + RN);             // fragment reads per K step
    auto frag_op = [&](auto dtag, const u32x4 *st, int ks, u32x4 (&al)[RM], u32x4 (&ah)[RM], u32x4 (&bl)[RN],
                       u32x4 (&bh)[RN]) {
        constexpr int d = decltype(dtag)::value;
        if constexpr (d < 2 * RM) {
            constexpr int i = d / 2, h = d % 2;
            (h ? ah : al)[i] = st[a_b[ks][h] + i * 32 * KG];
        } else {
            constexpr int j = (d - 2 * RM) / 2, h = (d - 2 * RM) % 2;
            (h ? bh : bl)[j] = st[A_SLOTS + b_b[ks][h] + j * 32 * KG];
        }
    };

    f32x16 acc[RM][RN];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    u32x4 al[2][RM], ah[2][RM], bl[2][RN], bh[2][RN];
    constexpr int NPR = (RM + RN) / 2;             // packed scale registers
    int sc[NPR];
#pragma unroll
    for (int e = 0; e < NPR; ++e) sc[e] = 0x7f7f7f7f;   // every byte: scale 1

    // The block-scale operands of K tile kt: read from LDS with the last
    // slice of the previous iteration (or after the first barrier), packed
    // at the start of the tile's iteration.  Blocks past the end of K (in
    // the last tile) get scale 1 -- their operands are zero, and those bytes
    // are not part of the caller's scale rows -- as does an operand without
    // block scales.
    const bool has_xa = p.xa != nullptr, has_xb = p.xb != nullptr;
    const uint32_t perm_sel = 0x06020400u + 0x01010101u * (uint32_t)fg;
    uint32_t raw[BSCALE ? RM + RN : 1];
    auto scale_read = [&](int kt) {
        if constexpr (BSCALE) {
            const uint32_t *sg = scale_ptr(kt);
#pragma unroll
            for (int e = 0; e < RM + RN; ++e) raw[e] = e < RM ? sg[sa_w + 128 * e] : sg[sb_w + 128 * (e - RM)];
        }
    };
    auto scales_for = [&](int kt) {
        if constexpr (BSCALE) {
            // (uniform masks of the bytes to keep: one bit-field insert each)
            const int rem = nkb - 4 * kt;
            const uint32_t keep = rem >= 4 ? 0xffffffffu : (rem <= 0 ? 0u : ((1u << (8 * rem)) - 1u));
            const uint32_t keep_a = has_xa ? keep : 0u;
            const uint32_t keep_b = has_xb ? keep : 0u;
#pragma unroll
            for (int e = 0; e < RM + RN; ++e) {
                const uint32_t k = e < RM ? keep_a : keep_b;
                raw[e] = (raw[e] & k) | (0x7f7f7f7fu & ~k);
            }
            // bytes (g, 2+g) of fragment 2p -> (0, 2), of fragment 2p+1 -> (1, 3)
#pragma unroll
            for (int e = 0; e < NPR; ++e) sc[e] = (int)__builtin_amdgcn_perm(raw[2 * e + 1], raw[2 * e], perm_sel);
        }
    };

    if (nk > 0) {
        static_for<0, STAGES>([&](auto s) { issue_to(decltype(s)::value, smem + decltype(s)::value * STAGE); });
        wait_vm_lgkm0<(STAGES - 1) * NDMA>();
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        static_for<0, NFR>([&](auto d) { frag_op(d, smem, 0, al[0], ah[0], bl[0], bh[0]); });
        scale_read(0);
    }

    // One K tile per iteration, as in the 16-bit kernel: step 0's MFMAs with
    // step 1's fragment reads, the barrier, then step 1's MFMAs interleaved
    // with the next tile's step-0 fragment (and scale) reads and the refill
    // of the stage just consumed.
    constexpr int NMF = RM * RN;
    int s_cur = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const int s_nxt = (s_cur + 1 == STAGES) ? 0 : s_cur + 1;
        u32x4 *cur = smem + s_cur * STAGE;
        u32x4 *nxt = smem + s_nxt * STAGE;
        scales_for(kt);
        static_for<0, NFR>([&](auto d) { frag_op(d, cur, 1, al[1], ah[1], bl[1], bh[1]); });
        static_for<0, NMF>([&](auto m) {
            constexpr int i = decltype(m)::value / RN, j = decltype(m)::value % RN;
            acc[i][j] = mfma_f8<FB, FA, j % 2, i % 2>(bl[0][j], bh[0][j], al[0][i], ah[0][i], acc[i][j],
                                                      sc[RM / 2 + j / 2], sc[i / 2]);
        });
        interleave_hint<NMF, NFR>();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        wait_vm_lgkm0<(STAGES - 2) * NDMA>();
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        wave_priority<1>();
        constexpr int NSUB = NDMA;
        static_for<0, NSUB>([&](auto sub) {
            constexpr int s0 = decltype(sub)::value;
            static_for<s0 * NMF / NSUB, (s0 + 1) * NMF / NSUB>([&](auto m) {
                constexpr int i = decltype(m)::value / RN, j = decltype(m)::value % RN;
                acc[i][j] = mfma_f8<FB, FA, 2 + j % 2, 2 + i % 2>(bl[1][j], bh[1][j], al[1][i], ah[1][i], acc[i][j],
                                                                  sc[RM / 2 + j / 2], sc[i / 2]);
            });
            static_for<s0 * NFR / NSUB, (s0 + 1) * NFR / NSUB>(
                [&](auto d) { frag_op(d, nxt, 0, al[0], ah[0], bl[0], bh[0]); });
            if constexpr (s0 == 0) scale_group(kt + STAGES);
            if constexpr (s0 == NSUB - 1) scale_read(kt + 1);
            dma_op(sub, kt + STAGES, cur);
            __builtin_amdgcn_sched_barrier(0);
        });
        wave_priority<0>();
        s_cur = s_nxt;
    }
    __builtin_amdgcn_s_waitcnt(0);

    // ---- epilogue: row scales, fp32 -> output type, masked store ----
    // One 32-row block of the wave's sub-tile at a time goes through the
    // wave's own LDS region in fp32; each lane then reads back 4 consecutive
    // values of a row, multiplies them by the row's A scale and the columns'
    // B scales, converts (round to nearest even) and stores them.  Rows past
    // M and columns past N are never stored.
    constexpr int ES = (CT == OUT_F32) ? 4 : 2;
    constexpr int ROWB = WTN * 4 + 16;             // staged row: fp32, padded by 16 bytes
    constexpr int CPR = WTN / 4;                   // 4-column chunks per row
    constexpr int RPI = 64 / CPR;                  // rows per read-back instruction
    constexpr int NT = 32 / RPI;                   // read-back instructions per 32-row block
    static_assert(RPI * CPR == 64 && 32 % RPI == 0, "row chunks must tile a wave");
    static_assert(NW * 32 * ROWB <= STAGES * STAGE * 16, "epilogue staging fits in LDS");
    const char *Cbase = (const char *)p.C + ((int64_t)m0 * p.ldc + n0) * ES;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cbase);
    const bool vec_store = (n0 + BN <= N) && (((uintptr_t)p.C | (uintptr_t)(p.ldc * ES)) & 3) == 0;
    const int chunk = lane % CPR;
    const int cn = wave_n * WTN + chunk * 4;
    f32x4 colsc = {1.0f, 1.0f, 1.0f, 1.0f};
    if (p.sb != nullptr) {
#pragma unroll
        for (int r = 0; r < 4; ++r) colsc[r] = (n0 + cn + r < N) ? p.sb[(int64_t)(n0 + cn + r) * p.inc_sb] : 0.0f;
    }
    float rowsc[RM][NT];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int m = m0 + wave_m * WTM + i * 32 + t * RPI + lane / CPR;
            rowsc[i][t] = (p.sa != nullptr && m < M) ? p.sa[(int64_t)m * p.inc_sa] : 1.0f;
        }
    __builtin_amdgcn_s_barrier();                  // every wave is done with the stages
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    char *const region = reinterpret_cast<char *>(smem) + wave * 32 * ROWB;
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
        for (int j = 0; j < RN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                *reinterpret_cast<f32x4 *>(region + fr * ROWB + (32 * j + 8 * q + 4 * fg) * 4) = v;
            }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int row = t * RPI + lane / CPR;
            f32x4 v = *reinterpret_cast<const f32x4 *>(region + row * ROWB + chunk * 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = (v[r] * rowsc[i][t]) * colsc[r];
            const int cm = wave_m * WTM + i * 32 + row;
            const bool row_ok = m0 + cm < M;
            if (vec_store) {
                const uint32_t off = row_ok ? (uint32_t)(cm * p.ldc + cn) * ES : OOB_OFFSET;
                if constexpr (CT == OUT_F32) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rc, off, 0, STORE_NT);
                    store_data_read(v);
                } else {
                    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                    u32x2 w;
                    if constexpr (CT == OUT_F16) {
                        w[0] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[0]) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[1]) << 16);
                        w[1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2]) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[3]) << 16);
                    } else {
                        w[0] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[0]) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[1]) << 16);
                        w[1] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2]) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[3]) << 16);
                    }
                    __builtin_amdgcn_raw_buffer_store_b64(w, rc, off, 0, STORE_NT);
                    store_data_read(w);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t off = (row_ok && n0 + cn + r < N) ? (uint32_t)(cm * p.ldc + cn + r) * ES : OOB_OFFSET;
                    if constexpr (CT == OUT_F32) {
                        // (the words of the whole vector: hipcc's bit cast of a
                        // single vector element reads element 0 whatever the index)
                        const uint32_t x = __builtin_bit_cast(u32x4, v)[r];
                        __builtin_amdgcn_raw_buffer_store_b32(x, rc, off, 0, STORE_NT);
                        store_data_read(x);
                    } else if constexpr (CT == OUT_F16) {
                        const uint16_t x = __builtin_bit_cast(uint16_t, (_Float16)v[r]);
                        __builtin_amdgcn_raw_buffer_store_b16(x, rc, off, 0, STORE_NT);
                        store_data_read(x);
                    } else {
                        const uint16_t x = __builtin_bit_cast(uint16_t, (__bf16)v[r]);
                        __builtin_amdgcn_raw_buffer_store_b16(x, rc, off, 0, STORE_NT);
                        store_data_read(x);
                    }
                }
            }
        }
        if (i + 1 < RM) __builtin_amdgcn_wave_barrier();   // the region is rewritten by the next block
    }
}

}  // namespace tdg
