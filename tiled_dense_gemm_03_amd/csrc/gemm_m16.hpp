// gemm_m16.hpp -- MFMA 16x16x32 GEMM kernel for gfx950 (aligned operands).
//
// The same decomposition as the other kernels (one workgroup per output
// tile, the K loop inside the workgroup, fp32 accumulators; NineToothed GEMM
// primer s4 and s6), built for large wave tiles:
//
//  * v_mfma_f32_16x16x32_{f16,bf16}.  Lane l supplies row l % 16 of an
//    operand and the 8 consecutive k values 8*(l / 16) .. +7; the 4 results
//    of lane l are rows 4*(l / 16) + r (r = 0..3) of column l % 16.  The
//    kernel passes the B fragment as the first operand, so lane l ends with
//    C[m = l % 16][n = 4*(l / 16) + r]: four consecutive output columns.
//    4-register accumulators leave the register allocator free to place a
//    128 x 128 wave tile (256 accumulator registers) in AccVGPRs.
//  * Direct global -> LDS loads (buffer_load_dwordx4 ... lds) as in the
//    other direct-load kernel, with leaner addressing: every load of a wave
//    uses one of at most two per-lane byte offsets plus a uniform row offset,
//    and rows past the matrix edge are cut off by the buffer's record count
//    (the descriptor of each K tile ends at the last valid element), so the
//    per-lane state is a handful of registers whatever the tile size.  The
//    zero fill of out-of-range reads is the primer's s5 masked load.
//  * K-tail: a granule whose first k is at or past K gets an out-of-range
//    offset (A and TN-B); NN-B rows past K fall outside the record count.
//  * Either operand may be stored K-contiguous ("KC": A as M x K, B as N x K)
//    or K-strided ("MC": A as K x M, B as K x N).  A KC operand goes through
//    the K-contiguous LDS layout and 16-byte reads, an MC operand through the
//    transposing layout and reads described below for NN-B; the MFMA
//    fragments come out the same either way.
//
// LDS layouts (16-byte granules of 8 elements):
//   A, TN-B: [rows][8 granules], granule g of row r at r*8 + (g ^ ((r>>1)&7)).
//            The 16 rows read at once by 16 lanes (same granule) land on 16
//            distinct 16-byte bank groups; rows 16 apart share the pattern,
//            so one base address per K step serves every fragment.
//   NN-B:    [64 k][BN/8 granules], granule c of row k at
//            k*BN/8 + (c ^ (4*(k&3) + 2*((k>>3)&1))).  A transposing read
//            (ds_read_b64_tr_b16) touches 4 consecutive k rows and 2
//            granules per 16 lanes; the 32 lanes of one LDS cycle take
//            k rows 8 apart, which the (k>>3) term separates.
// Writer and reader derive positions from the same functions (the Croqtile
// tutorial ch.4 remarks that a swizzled store and the operand load must
// agree on the swizzle).
#pragma once

#include "gemm_fast.hpp"

namespace tdg {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int AB>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (AB == AB_F16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
}

// The same MFMA as inline assembly with the accumulator tied to AccVGPRs
// (the "+a" operand is both source C and destination).  Used when a wave's
// accumulators outgrow the VGPRs: hipcc then mixes register classes for the
// intrinsic and copies accumulators between them on every K step.  The
// compiler does not know the statement is an MFMA, so its users (i) order
// it by hand (sched_barrier; IGroupLP cannot classify it), (ii) wait out the
// MFMA result latency before any other instruction reads an accumulator
// (mfma_asm_drain) and (iii) keep the zero initialisation of the
// accumulators apart from the first MFMA (mfma_asm_pin).
template <int AB>
__device__ __forceinline__ f32x4 mfma_16x16x32_acc(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (AB == AB_F16) {
        asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    } else {
        asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
    return c;
}
__device__ __forceinline__ void mfma_asm_pin(f32x4 &c) { asm volatile("" : "+a"(c)); }

// Direct 16-byte load to LDS address lds_base + IMM with M0 as an operand of
// the statement (one scalar move per load instead of saving and restoring
// M0 around it).
template <uint32_t IMM>
__device__ __forceinline__ void dma16_m0(u32x4 rsrc, uint32_t voff, uint32_t lds_base) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base + IMM) : "memory");
}
template <bool M0_OPERAND, uint32_t IMM>
__device__ __forceinline__ void dma16_sel(u32x4 rsrc, uint32_t voff, uint32_t lds_base) {
    if constexpr (M0_OPERAND) dma16_m0<IMM>(rsrc, voff, lds_base);
    else dma16<IMM>(rsrc, voff, lds_base);
}
// 32 wait states: more than the 8-pass MFMA's result latency for any reader.
__device__ __forceinline__ void mfma_asm_drain() { asm volatile("s_nop 15\n\ts_nop 15" ::: "memory"); }

// This wave's issue priority among the waves of its SIMD (0 or 1), fenced
// so the compiler keeps the surrounding instructions on their side.  Raised
// for the second half of each K tile (MFMAs interleaved with fragment reads
// and the stage refill) in the K-contiguous-B kernels: measured +3.5% on
// 8192^3 TN with fp32 output and +2 to +3.5% on the 8-bit kernel, while the
// NN form and the persistent kernel gain nothing from it.
template <int PRIO>
__device__ __forceinline__ void wave_priority() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(PRIO);
    __builtin_amdgcn_sched_barrier(0);
}

// Buffer descriptor words with an explicit record count (bytes).
__device__ __forceinline__ u32x4 rsrc_words_n(const void *base, uint32_t records) {
    const uint64_t a = (uint64_t)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    r[2] = __builtin_amdgcn_readfirstlane(records);
    r[3] = (uint32_t)BUF_FLAGS;
    return r;
}

// Record count for `elems` valid elements (clamped to [0, 2^31 - 1]).
__device__ __forceinline__ uint32_t records_of(int64_t elems) {
    const int64_t b = elems * 2;
    return b <= 0 ? 0u : (b >= (int64_t)BUF_RECORDS ? (uint32_t)BUF_RECORDS : (uint32_t)b);
}

__device__ __forceinline__ int kx16(int r) { return (r >> 1) & 7; }                 // K-contiguous XOR
// The same for K tiles of 32 (rows of 4 granules): the 16 rows read at once
// by 16 lanes land on 16 distinct 16-byte bank groups.
template <int KG>
__device__ __forceinline__ int kxor(int r) { return KG == 8 ? (r >> 1) & 7 : (r >> 2) & 3; }
__device__ __forceinline__ int nx16(int k) { return 4 * (k & 3) + 2 * ((k >> 3) & 1); }  // NN-B XOR

// BM x BN workgroup tile, WM x WN waves of (BM/WM) x (BN/WN), K tiles of 64
// (BKT = 32: of 32) in STAGES LDS stages.
//
// TRANSA: false = A stored M x K (KC), true = A stored K x M (MC).
// TRANSB: false = B stored K x N (MC), true = B stored N x K (KC).
// PP: the ping-pong schedule (two wave groups alternating memory and MFMA
// phases).  AWIN: the A window (A rows loaded as line-aligned chunks into a
// ring of three slots, for rows that do not start on 128-byte lines).
template <int BM, int BN, int WM, int WN, int STAGES, bool TRANSA, bool TRANSB, int AB, int CT, bool PP = false,
          int BKT = 64, bool AWIN = false>
__global__ __launch_bounds__(WM * WN * 64) void gemm_m16_kernel(GemmArgs p) {
    constexpr int BK = BKT, KS = BK / 32, KG = BK / GRAN, BNG = BN / GRAN, BMG = BM / GRAN;
    static_assert(BK == 64 || (BK == 32 && !PP), "K tiles of 64, or of 32 (one MFMA K step per stage)");
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int RM = WTM / 16, RN = WTN / 16;
    static_assert(RM * 16 == WTM && RN * 16 == WTN, "wave tile must be a multiple of 16");
    static_assert(NW % 2 == 0, "an even number of waves");
    static_assert(TRANSB || (BNG >= 16 && (BNG & (BNG - 1)) == 0), "MC B rows: a power of two >= 16 granules");
    static_assert(!TRANSA || (BMG >= 16 && (BMG & (BMG - 1)) == 0), "MC A rows: a power of two >= 16 granules");
    constexpr int A_SLOTS = BM * KG, B_SLOTS = BN * KG, STAGE = A_SLOTS + B_SLOTS;
    constexpr int NIA = A_SLOTS / 64, NIB = B_SLOTS / 64;
    static_assert(NIA % NW == 0 && NIB % NW == 0, "whole load instructions per wave");
    constexpr int QA = NIA / NW, QB = NIB / NW, NDMA = QA + QB;
    static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 stages");
    static_assert(BK == 64 || STAGES >= 3, "K tiles of 32 run at least two stages ahead");
    static_assert((STAGES - 1) * NDMA < 64, "vmcnt range");
    static_assert(STAGE * 16 * STAGES <= 160 * 1024, "LDS budget");
    // An MC load instruction t covers k rows t*RP .. +RP-1 (RP = 64 granules
    // / granules per k row); its XOR pattern repeats every NV instructions of
    // one wave (NV = 16 / gcd(16, NW * RP)).
    constexpr int RPB = 64 / BNG, RPA = 64 / BMG;
    constexpr int NVB = TRANSB ? 1 : 16 / ((NW * RPB) % 16 == 0 ? 16 : ((NW * RPB) % 8 == 0 ? 8 : ((NW * RPB) % 4 == 0 ? 4 : ((NW * RPB) % 2 == 0 ? 2 : 1))));
    constexpr int NVA = !TRANSA ? 1 : 16 / ((NW * RPA) % 16 == 0 ? 16 : ((NW * RPA) % 8 == 0 ? 8 : ((NW * RPA) % 4 == 0 ? 4 : ((NW * RPA) % 2 == 0 ? 2 : 1))));

    // Accumulators beyond 160 registers per lane (a 4-wave 128 x 128 wave
    // tile has 256) are kept in AccVGPRs by the tied inline-assembly MFMA.
    constexpr bool ASM_ACC = (BM / WM / 16) * (BN / WN / 16) * 4 > 160;
    static_assert(!PP || (WM == 2 && WN == 4 && STAGES == 2 && !ASM_ACC),
                  "the ping-pong schedule: two groups of four waves (one per SIMD each), two stages");
    // AWIN: A (stored M x K) whose rows do not start on 128-byte lines is
    // loaded as whole aligned 128-byte chunks of each row into a ring of
    // three A slots (B keeps two stages); see the A-window loop below.
    static_assert(!AWIN || (!TRANSA && BK == 64 && !PP && !ASM_ACC), "the A window: A stored M x K, K tiles of 64");
    constexpr int AW_R = STAGES + 1;                  // A chunk slots of the A window
    constexpr int LDS_SLOTS = AWIN ? AW_R * A_SLOTS + STAGES * B_SLOTS : STAGES * STAGE;
    static_assert(LDS_SLOTS * 16 <= 160 * 1024, "LDS budget");

    __shared__ u32x4 smem[LDS_SLOTS];
    auto stage_ptr = [&](auto tag) -> u32x4 * { return smem + decltype(tag)::value * STAGE; };

    // ---- work item: a whole tile, or one K slice of a split tile ----
    // Workgroups [0, dp_tiles) take the first dp_tiles tiles; the rest take
    // K slices of the remaining tiles, sk_split consecutive work items per
    // tile.  Each phase is spread over the XCDs on its own, so both the whole
    // tiles and the slices are balanced over the chip, and the slices of one
    // tile meet on one XCD.
    const int nk_all = (p.K + BK - 1) / BK;
    int batch, tm, tn, kt_begin = 0, kt_end = nk_all, slice = 0, split_tile = -1;
    {
        const int w = blockIdx.x, dp = p.dp_tiles;
        int logical;
        if (w < dp) {
            logical = xcd_order(w, dp);
        } else {
            const int u = xcd_order(w - dp, (int)gridDim.x - dp);
            split_tile = u / p.sk_split;
            slice = u - split_tile * p.sk_split;
            logical = dp + split_tile;
            kt_begin = (int)((int64_t)nk_all * slice / p.sk_split);
            kt_end = (int)((int64_t)nk_all * (slice + 1) / p.sk_split);
        }
        tile_of(p, logical, batch, tm, tn);
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave / WN, wave_n = wave % WN;
    const int M = p.M, N = p.N;
    // loads stop at the end of this work item's K range (the prefetches past
    // it read nothing)
    const int K = p.K < kt_end * BK ? p.K : kt_end * BK;
    const int m0 = tm * BM, n0 = tn * BN;
    const int64_t lda = p.lda, ldb = p.ldb;

    const uint16_t *Atile = TRANSA ? p.A + (int64_t)batch * p.sA + m0
                                   : p.A + (int64_t)batch * p.sA + (int64_t)m0 * lda;
    const uint16_t *Btile = TRANSB ? p.B + (int64_t)batch * p.sB + (int64_t)n0 * ldb
                                   : p.B + (int64_t)batch * p.sB + n0;
    const int a_rows = M - m0 < BM ? M - m0 : BM;
    const int b_rows = N - n0 < BN ? N - n0 : BN;     // TN: valid B rows; NN: valid columns

    // ---- direct-load addressing ----
    // K-contiguous operand, load q of this wave = instruction t = q*NW + wave:
    // LDS slots 64t .. 64t+63 = rows RI*t .. RI*t+RI-1 of KG granules (RI =
    // 64 / KG: 8 rows for K tiles of 64, 16 for 32).  The lane's row is
    // RI*t + lane/KG and its granule g = (lane%KG) ^ kxor(row); kxor does not
    // depend on q (NW is even), so the byte offset is a_lane + q*a_qs.
    constexpr int RI = 64 / KG;
    const int kc_row = wave * RI + lane / KG;
    const int kc_g = (lane % KG) ^ kxor<KG>(kc_row);
    const int kc_klim = K - kc_g * GRAN;           // granule loaded while k0 < kc_klim
    uint32_t a_lane[NVA];
    uint32_t a_qs;
    if constexpr (!TRANSA) {
        a_lane[0] = (uint32_t)((kc_row * lda + kc_g * GRAN) * 2);
        a_qs = (uint32_t)(NW * RI * lda * 2);
    } else {
        // MC A: as MC B below, with M for N
#pragma unroll
        for (int v = 0; v < NVA; ++v) {
            const int kr = RPA * wave + lane / BMG;
            const int k = RPA * (v * NW) + kr;
            const int c = (lane % BMG) ^ nx16(k);
            a_lane[v] = (m0 + c * GRAN < M) ? (uint32_t)((kr * lda + c * GRAN) * 2) : OOB_OFFSET;
        }
        a_qs = (uint32_t)(NW * RPA * lda * 2);
    }
    uint32_t b_lane[NVB];
    uint32_t b_qs;
    if constexpr (TRANSB) {
        b_lane[0] = (uint32_t)((kc_row * ldb + kc_g * GRAN) * 2);
        b_qs = (uint32_t)(NW * RI * ldb * 2);
    } else {
        // NN-B instruction t covers k rows RPB*t .. ; the lane's k is
        // RPB*t + lane / BNG and its column granule (lane % BNG) ^ nx16(k).
#pragma unroll
        for (int v = 0; v < NVB; ++v) {
            const int kr = RPB * wave + lane / BNG;          // k row relative to instruction q = 0
            const int k = RPB * (v * NW) + kr;
            const int c = (lane % BNG) ^ nx16(k);
            b_lane[v] = (n0 + c * GRAN < N) ? (uint32_t)((kr * ldb + c * GRAN) * 2) : OOB_OFFSET;
        }
        b_qs = (uint32_t)(NW * RPB * ldb * 2);
    }

    auto dma_op = [&](auto qtag, int kt, u32x4 *sa) {
        constexpr int q = decltype(qtag)::value;
        const int k0 = kt * BK;
        const uint32_t base = lds_addr_of(sa) + (uint32_t)wave * 1024u;
        if constexpr (q < QA) {
            if constexpr (!TRANSA) {
                const u32x4 rs = rsrc_words_n(Atile + k0, records_of((int64_t)(a_rows - 1) * lda + K - k0));
                const uint32_t off = (k0 < kc_klim ? a_lane[0] : OOB_OFFSET) + (uint32_t)q * a_qs;
                dma16_sel<ASM_ACC, (uint32_t)(q * NW) * 1024u>(rs, off, base);
            } else {
                const u32x4 rs = rsrc_words_n(Atile + (int64_t)k0 * lda,
                                              records_of((int64_t)(K - k0 - 1) * lda + (M - m0)));
                const uint32_t off = a_lane[q % NVA] + (uint32_t)q * a_qs;
                dma16_sel<ASM_ACC, (uint32_t)(q * NW) * 1024u>(rs, off, base);
            }
        } else {
            constexpr int qb = q - QA;
            if constexpr (TRANSB) {
                const u32x4 rs = rsrc_words_n(Btile + k0, records_of((int64_t)(b_rows - 1) * ldb + K - k0));
                const uint32_t off = (k0 < kc_klim ? b_lane[0] : OOB_OFFSET) + (uint32_t)qb * b_qs;
                dma16_sel<ASM_ACC, (uint32_t)(A_SLOTS * 16 + qb * NW * 1024)>(rs, off, base);
            } else {
                const u32x4 rs = rsrc_words_n(Btile + (int64_t)k0 * ldb,
                                              records_of((int64_t)(K - k0 - 1) * ldb + (N - n0)));
                const uint32_t off = b_lane[qb % NVB] + (uint32_t)qb * b_qs;
                dma16_sel<ASM_ACC, (uint32_t)(A_SLOTS * 16 + qb * NW * 1024)>(rs, off, base);
            }
        }
    };
    auto issue_to = [&](int kt, u32x4 *sa) { static_for<0, NDMA>([&](auto q) { dma_op(q, kt, sa); }); };

    // ---- fragment addresses ----
    // A (and TN-B) fragment i at K step ks: row wave_x*WT + 16 i + lane%16,
    // granule 4 ks + lane/16; kxor of that row is kxor(lane%16) for every i
    // (rows 16 apart share the pattern).
    const int fr = lane & 15, fg = lane >> 4;
    int a_b[KS], bt_b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        a_b[ks] = (wave_m * WTM + fr) * KG + ((4 * ks + fg) ^ kxor<KG>(fr));
        bt_b[ks] = (wave_n * WTN + fr) * KG + ((4 * ks + fg) ^ kxor<KG>(fr));
    }
    // NN-B fragment j, half h at K step ks: lane supplies the 8 bytes at k
    // row 32 ks + 8 fg + 4 h + jr, columns wave_n*WTN + 16 j + 4 q4 .. +3;
    // nx16 of that row is 4 jr + 2 (fg & 1) for every (ks, h), so (ks, h)
    // are constant offsets.
    const int jr = (lane & 15) >> 2, q4 = lane & 3;
    int bn_b[TRANSB ? 1 : RN];
    if constexpr (!TRANSB) {
#pragma unroll
        for (int j = 0; j < RN; ++j) {
            const int c = (wave_n * WTN + 16 * j + 4 * q4) / GRAN;
            bn_b[j] = ((8 * fg + jr) * BNG + (c ^ (4 * jr + 2 * (fg & 1)))) * 16 + (q4 & 1) * 8;
        }
    }
    int am_b[TRANSA ? RM : 1];
    if constexpr (TRANSA) {
#pragma unroll
        for (int i = 0; i < RM; ++i) {
            const int c = (wave_m * WTM + 16 * i + 4 * q4) / GRAN;
            am_b[i] = ((8 * fg + jr) * BMG + (c ^ (4 * jr + 2 * (fg & 1)))) * 16 + (q4 & 1) * 8;
        }
    }

    // LDS reads of an MC operand: two transposing 8-byte reads (k rows
    // 0..3 and 4..7 of the lane's run) fill one fragment.
    auto tr_read = [&](const u32x4 *st, int byte_off, u32x4 &frag, auto htag) {
        constexpr int h = decltype(htag)::value;
        const char *base = reinterpret_cast<const char *>(st);
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(base + byte_off));
        const uint64_t w = __builtin_bit_cast(uint64_t, v);
        frag[2 * h] = (uint32_t)w;
        frag[2 * h + 1] = (uint32_t)(w >> 32);
    };
    constexpr int DA = TRANSA ? 2 * RM : RM;     // LDS reads for the A fragments of one K step
    auto frag_op = [&](auto dtag, const u32x4 *sa, int ks, u32x4 (&af)[RM], u32x4 (&bf)[RN]) {
        constexpr int d = decltype(dtag)::value;
        const u32x4 *sb = sa + A_SLOTS;
        if constexpr (d < DA) {
            if constexpr (!TRANSA) {
                af[d] = sa[a_b[ks] + d * 16 * KG];
            } else {
                constexpr int i = d / 2, h = d % 2;
                tr_read(sa, am_b[i] + (32 * ks + 4 * h) * BMG * 16, af[i], std::integral_constant<int, h>{});
            }
        } else if constexpr (TRANSB) {
            constexpr int j = d - DA;
            bf[j] = sb[bt_b[ks] + j * 16 * KG];
        } else {
            constexpr int j = (d - DA) / 2, h = (d - DA) % 2;
            tr_read(sb, bn_b[j] + (32 * ks + 4 * h) * BNG * 16, bf[j], std::integral_constant<int, h>{});
        }
    };
    constexpr int NDS = DA + (TRANSB ? RN : 2 * RN);
    constexpr int NMF = RM * RN;
    auto frags_from = [&](const u32x4 *sa, int ks, u32x4 (&af)[RM], u32x4 (&bf)[RN]) {
        static_for<0, NDS>([&](auto d) { frag_op(d, sa, ks, af, bf); });
    };

    f32x4 acc[RM][RN];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j) {
            acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (ASM_ACC) mfma_asm_pin(acc[i][j]);
        }

    u32x4 af[2][RM], bf[2][RN];

    if constexpr (PP) {
        // ---- ping-pong schedule: wave roles that alternate ----
        // Group g = wave_m (waves 0-3 and 4-7: one wave of each group per
        // SIMD).  Each K tile t is a memory phase -- this wave's share of the
        // direct loads of tile t+1 into the other stage, then all of tile
        // t's operand fragments from LDS into registers -- then a barrier,
        // then a compute phase of nothing but the tile's 64 MFMAs, then a
        // barrier.  Group 1 starts one phase late, so in every phase one
        // group computes while the other loads and reads: each SIMD's MFMA
        // pipe is fed by one wave while the other wave's memory work runs
        // beside it (the role split of the Croqtile tutorial, chapter 4,
        // last paragraph: a group that loads while another computes).
        // Stage reuse: tile t sits in stage t % 2 and is read by group 0 in
        // phase 2t and by group 1 in phase 2t+1; tile t+2 goes into that
        // stage during phases 2t+2 (group 0's share) and 2t+3 (group 1's),
        // after the barrier that ends phase 2t+1.  Group 0 waits for its
        // share at the end of its compute phase 2t+3, group 1 at the end of
        // its memory phase 2t+3, so tile t+2 is complete at the barrier
        // before phase 2t+4, where group 0 first reads it.  The MFMAs run in
        // the order of the other schedules, so the sums are the same bits.
        const int g = wave_m;
        const int nkt = kt_end - kt_begin;
        if (nkt > 0) {
            issue_to(kt_begin, smem);
            wait_vm_lgkm0<0>();
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        if (g == 1) __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        for (int t = 0; t < nkt; ++t) {
            u32x4 *cur = smem + (t & 1) * STAGE;
            u32x4 *nxt = smem + ((t + 1) & 1) * STAGE;
            // memory phase
            issue_to(kt_begin + t + 1, nxt);
            frags_from(cur, 0, af[0], bf[0]);
            frags_from(cur, 1, af[1], bf[1]);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (g == 1) wait_vm_lgkm0<0>();
            else wait_vm_lgkm0<NDMA>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // compute phase
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int i = 0; i < RM; ++i)
#pragma unroll
                    for (int j = 0; j < RN; ++j) acc[i][j] = mfma_16x16x32<AB>(bf[ks][j], af[ks][i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
            if (g == 0) wait_vm_lgkm0<0>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
        if (g == 0) __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    } else if (!AWIN && kt_end > kt_begin) {
        static_for<0, STAGES>([&](auto s) { issue_to(kt_begin + decltype(s)::value, stage_ptr(s)); });
        // K tiles of 64: the first stage; of 32: the first two (the second
        // one's fragments are read during the first step)
        wait_vm_lgkm0<(BK == 32 ? STAGES - 2 : STAGES - 1) * NDMA>();
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        frags_from(smem, 0, af[0], bf[0]);
    }

    // One K tile per iteration, held in stage s_cur: step 0 (its MFMAs with
    // step 1's fragment reads), then the barrier, then step 1's MFMAs
    // interleaved with the next tile's step-0 fragment reads and the refill
    // of stage s_cur.  The stage is a run-time index (one loop body, no
    // per-stage copies of the code).
    int s_cur = 0;
    if constexpr (PP) {
        // (the ping-pong loop ran above)
    } else if constexpr (AWIN) {
        // ---- A window: rows of A that do not start on a 128-byte line ----
        // A row whose K run of a tile (128 bytes) starts s bytes past a line
        // boundary touches two lines per load instruction instead of one.
        // Here each row is loaded as its own aligned 128-byte chunks instead:
        // chunk c of row r holds the bytes [128 c, 128 c + 128) of the row's
        // line-aligned stream, i.e. elements 64 c - s/2 .. 64 c - s/2 + 63.
        // Tile kt's elements of the row then lie in chunks kt and kt + 1, so
        // STAGES + 1 chunk slots make a ring: chunks kt, kt + 1 in use,
        // kt + 2 .. kt + STAGES arriving, and chunk kt + STAGES + 1 loaded
        // into chunk kt's slot once tile kt is read (with B tile kt + STAGES
        // into tile kt's B stage).  The shift s is a multiple of 16 bytes
        // (lda is a multiple of 8) and depends on the row only modulo 8, so
        // every lane has one shift for its loads and one for its fragment
        // reads.  Elements before the row's first or past its K-th read as
        // zeros.  LDS: A slot c % (STAGES + 1), then the B stages.  Within a
        // chunk slot, granule g of row r (shift d = s / 16 granules) sits at
        // ((g - d) & 7) ^ kx16(r): rotated by the row's shift, so that the
        // granule a fragment read wants (4 ks + lane / 16 + d of the window,
        // in chunk kt or kt + 1) is at (4 ks + lane / 16) ^ kx16(r) whatever
        // d is -- the positions of the plain layout, whose reads do not
        // conflict (unrotated, rows of different shifts put 25x the bank
        // conflict cycles on the fragment reads).
        const char *Abytes = reinterpret_cast<const char *>(Atile);
        const int s_ld = (int)(((uintptr_t)Abytes + (uintptr_t)(kc_row * lda * 2)) & 127);
        const int aw_g = (((lane % KG) ^ kxor<KG>(kc_row)) + (s_ld >> 4)) & 7;   // chunk granule this lane loads
        const int aw_e0 = 8 * aw_g - s_ld / 2;          // element of the lane's granule in chunk 0
        const uint32_t aw_off = (uint32_t)(kc_row * lda * 2 + 16 * aw_g - s_ld + 128);
        const int d_rd = (int)((((uintptr_t)Abytes + (uintptr_t)(fr * lda * 2)) & 127) >> 4);
        int aw_b[KS], aw_co[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            aw_co[ks] = (4 * ks + fg + d_rd) >> 3;        // chunk kt or kt + 1
            aw_b[ks] = (wave_m * WTM + fr) * KG + ((4 * ks + fg) ^ kxor<KG>(fr));
        }
        u32x4 *const bstages = smem + AW_R * A_SLOTS;
        auto dma_a = [&](auto qtag, int c) {              // A chunk c into slot c % AW_R
            constexpr int q = decltype(qtag)::value;
            const uint32_t base = lds_addr_of(smem + (c % AW_R) * A_SLOTS) + (uint32_t)wave * 1024u;
            const u32x4 rs = rsrc_words_n(Abytes + 128 * (int64_t)(c - 1),
                                          records_of(64 * (int64_t)(1 - c) + (int64_t)(a_rows - 1) * lda + K));
            const int e = 64 * c + aw_e0;
            const uint32_t off = (e >= 0 && e + GRAN <= K) ? aw_off + (uint32_t)q * a_qs : OOB_OFFSET;
            dma16_sel<false, (uint32_t)(q * NW) * 1024u>(rs, off, base);
        };
        auto dma_b = [&](auto qtag, int kt, u32x4 *bst) {  // B load qb of K tile kt into a B stage
            constexpr int qb = decltype(qtag)::value;
            const int k0 = kt * BK;
            const uint32_t base = lds_addr_of(bst) + (uint32_t)wave * 1024u;
            if constexpr (TRANSB) {
                const u32x4 rs = rsrc_words_n(Btile + k0, records_of((int64_t)(b_rows - 1) * ldb + K - k0));
                const uint32_t off = (k0 < kc_klim ? b_lane[0] : OOB_OFFSET) + (uint32_t)qb * b_qs;
                dma16_sel<false, (uint32_t)(qb * NW * 1024)>(rs, off, base);
            } else {
                const u32x4 rs = rsrc_words_n(Btile + (int64_t)k0 * ldb,
                                              records_of((int64_t)(K - k0 - 1) * ldb + (N - n0)));
                const uint32_t off = b_lane[qb % NVB] + (uint32_t)qb * b_qs;
                dma16_sel<false, (uint32_t)(qb * NW * 1024)>(rs, off, base);
            }
        };
        // K step ks of tile kt (chunks kt, kt + 1; B stage bst): fragment d
        auto frag_w = [&](auto dtag, int kt, const u32x4 *bst, int ks, u32x4 (&af)[RM], u32x4 (&bf)[RN]) {
            constexpr int d = decltype(dtag)::value;
            if constexpr (d < RM) {
                const int slot = (kt + aw_co[ks]) % AW_R;
                af[d] = smem[slot * A_SLOTS + aw_b[ks] + d * 16 * KG];
            } else {
                frag_op(dtag, bst - A_SLOTS, ks, af, bf);  // (frag_op reads B at its argument + A_SLOTS)
            }
        };
        if (kt_end > kt_begin) {
            // chunks kt_begin, kt_begin + 1 and B tile kt_begin first, then
            // for each later stage s, chunk kt_begin + s + 1 and B tile
            // kt_begin + s; the first group is waited for
            static_for<0, QA>([&](auto q) { dma_a(q, kt_begin); });
            static_for<0, QA>([&](auto q) { dma_a(q, kt_begin + 1); });
            static_for<0, QB>([&](auto q) { dma_b(q, kt_begin, bstages); });
            static_for<1, STAGES>([&](auto st) {
                constexpr int sg = decltype(st)::value;
                static_for<0, QA>([&](auto q) { dma_a(q, kt_begin + sg + 1); });
                static_for<0, QB>([&](auto q) { dma_b(q, kt_begin + sg, bstages + sg * B_SLOTS); });
            });
            wait_vm_lgkm0<(STAGES - 1) * NDMA>();
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            static_for<0, NDS>([&](auto d) { frag_w(d, kt_begin, bstages, 0, af[0], bf[0]); });
        }
        int b_cur = 0;
        for (int kt = kt_begin; kt < kt_end; ++kt) {
            const int b_nxt = (b_cur + 1 == STAGES) ? 0 : b_cur + 1;
            u32x4 *bcur = bstages + b_cur * B_SLOTS;
            u32x4 *bnxt = bstages + b_nxt * B_SLOTS;
            static_for<0, NDS>([&](auto d) { frag_w(d, kt, bcur, 1, af[1], bf[1]); });
#pragma unroll
            for (int i = 0; i < RM; ++i)
#pragma unroll
                for (int j = 0; j < RN; ++j) acc[i][j] = mfma_16x16x32<AB>(bf[0][j], af[0][i], acc[i][j]);
            interleave_hint<NMF, NDS>();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            wait_vm_lgkm0<(STAGES - 2) * NDMA>();
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if constexpr (TRANSB) wave_priority<1>();
            constexpr int NSUB = NDMA;
            static_for<0, NSUB>([&](auto sub) {
                constexpr int s0 = decltype(sub)::value;
                static_for<s0 * NMF / NSUB, (s0 + 1) * NMF / NSUB>([&](auto m) {
                    constexpr int i = decltype(m)::value / RN, j = decltype(m)::value % RN;
                    acc[i][j] = mfma_16x16x32<AB>(bf[1][j], af[1][i], acc[i][j]);
                });
                static_for<s0 * NDS / NSUB, (s0 + 1) * NDS / NSUB>(
                    [&](auto d) { frag_w(d, kt + 1, bnxt, 0, af[0], bf[0]); });
                if constexpr (s0 < QA) dma_a(sub, kt + STAGES + 1);
                else dma_b(std::integral_constant<int, s0 - QA>{}, kt + STAGES, bcur);
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (TRANSB) wave_priority<0>();
            b_cur = b_nxt;
        }
    } else if constexpr (BK == 32) {
        // K tiles of 32: one MFMA K step per stage and one barrier per step.
        // Step kt's MFMAs run interleaved with the fragment reads of step
        // kt+1 and the direct loads of step kt+STAGES into the stage step kt
        // occupied (its fragments were read before the previous barrier),
        // so the loads of every step are spread over a whole step, and run
        // STAGES steps ahead.  The wait before each barrier leaves STAGES-2
        // steps of loads in flight: step kt+2, read during step kt+1, has
        // landed.  Two steps per loop pass, for the two fragment buffers.
        auto step = [&](int kt, auto xtag) {
            constexpr int x = decltype(xtag)::value;
            const int s_nxt = (s_cur + 1 == STAGES) ? 0 : s_cur + 1;
            u32x4 *cur = smem + s_cur * STAGE;
            u32x4 *nxt = smem + s_nxt * STAGE;
            constexpr int NSUB = NDMA;
            static_for<0, NSUB>([&](auto sub) {
                constexpr int s0 = decltype(sub)::value;
                static_for<s0 * NMF / NSUB, (s0 + 1) * NMF / NSUB>([&](auto m) {
                    constexpr int i = decltype(m)::value / RN, j = decltype(m)::value % RN;
                    acc[i][j] = mfma_16x16x32<AB>(bf[x][j], af[x][i], acc[i][j]);
                });
                static_for<s0 * NDS / NSUB, (s0 + 1) * NDS / NSUB>(
                    [&](auto d) { frag_op(d, nxt, 0, af[1 - x], bf[1 - x]); });
                dma_op(sub, kt + STAGES, cur);
                __builtin_amdgcn_sched_barrier(0);
            });
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            wait_vm_lgkm0<(STAGES - 2) * NDMA>();
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            s_cur = s_nxt;
        };
        for (int kt = kt_begin; kt < kt_end; kt += 2) {
            step(kt, std::integral_constant<int, 0>{});
            if (kt + 1 < kt_end) step(kt + 1, std::integral_constant<int, 1>{});
        }
    } else if constexpr (!ASM_ACC) {
        for (int kt = kt_begin; kt < kt_end; ++kt) {
            const int s_nxt = (s_cur + 1 == STAGES) ? 0 : s_cur + 1;
            u32x4 *cur = smem + s_cur * STAGE;
            u32x4 *nxt = smem + s_nxt * STAGE;
            frags_from(cur, 1, af[1], bf[1]);
#pragma unroll
            for (int i = 0; i < RM; ++i)
#pragma unroll
                for (int j = 0; j < RN; ++j) acc[i][j] = mfma_16x16x32<AB>(bf[0][j], af[0][i], acc[i][j]);
            interleave_hint<NMF, NDS>();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            wait_vm_lgkm0<(STAGES - 2) * NDMA>();
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if constexpr (TRANSB) wave_priority<1>();
            constexpr int NSUB = NDMA;
            static_for<0, NSUB>([&](auto sub) {
                constexpr int s0 = decltype(sub)::value;
                static_for<s0 * NMF / NSUB, (s0 + 1) * NMF / NSUB>([&](auto m) {
                    constexpr int i = decltype(m)::value / RN, j = decltype(m)::value % RN;
                    acc[i][j] = mfma_16x16x32<AB>(bf[1][j], af[1][i], acc[i][j]);
                });
                static_for<s0 * NDS / NSUB, (s0 + 1) * NDS / NSUB>([&](auto d) { frag_op(d, nxt, 0, af[0], bf[0]); });
                dma_op(sub, kt + STAGES, cur);
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (TRANSB) wave_priority<0>();
            s_cur = s_nxt;
        }
    } else {
        // The same schedule with every slice fenced by sched_barrier.  The
        // fragment reads go in the order the MFMAs consume them (A fragment
        // 0, every B fragment, then A fragments 1..), so that the MFMAs of
        // a step can start before all of its fragments have arrived.
        constexpr int PA = DA / RM, NB = NDS - DA;
        auto rd = [](auto ctag) {
            constexpr int c = decltype(ctag)::value;
            return std::integral_constant<int, (c < PA ? c : (c < PA + NB ? DA + (c - PA) : c - NB))>{};
        };
        for (int kt = kt_begin; kt < kt_end; ++kt) {
            const int s_nxt = (s_cur + 1 == STAGES) ? 0 : s_cur + 1;
            u32x4 *cur = smem + s_cur * STAGE;
            u32x4 *nxt = smem + s_nxt * STAGE;
            static_for<0, NDS>([&](auto c) {
                constexpr int c0 = decltype(c)::value;
                static_for<c0 * NMF / NDS, (c0 + 1) * NMF / NDS>([&](auto m) {
                    constexpr int i = decltype(m)::value / RN, j = decltype(m)::value % RN;
                    acc[i][j] = mfma_16x16x32_acc<AB>(bf[0][j], af[0][i], acc[i][j]);
                });
                frag_op(rd(c), cur, 1, af[1], bf[1]);
                __builtin_amdgcn_sched_barrier(0);
            });
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            wait_vm_lgkm0<(STAGES - 2) * NDMA>();
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            constexpr int NSUB = NDMA > NDS ? NDMA : NDS;
            static_for<0, NSUB>([&](auto sub) {
                constexpr int s0 = decltype(sub)::value;
                static_for<s0 * NMF / NSUB, (s0 + 1) * NMF / NSUB>([&](auto m) {
                    constexpr int i = decltype(m)::value / RN, j = decltype(m)::value % RN;
                    acc[i][j] = mfma_16x16x32_acc<AB>(bf[1][j], af[1][i], acc[i][j]);
                });
                static_for<s0 * NDS / NSUB, (s0 + 1) * NDS / NSUB>([&](auto c) { frag_op(rd(c), nxt, 0, af[0], bf[0]); });
                static_for<s0 * NDMA / NSUB, (s0 + 1) * NDMA / NSUB>([&](auto q) { dma_op(q, kt + STAGES, cur); });
                __builtin_amdgcn_sched_barrier(0);
            });
            s_cur = s_nxt;
        }
        mfma_asm_drain();
    }
    __builtin_amdgcn_s_waitcnt(0);

    // ---- split tiles: combine the K slices ----
    // Every slice stores its fp32 partial tile (each lane its own 16-byte
    // pieces, so each wave store is 1 KiB contiguous) and takes a ticket from
    // the tile's counter; the slice that draws the last ticket sums the
    // partials in slice order (the same rounding whichever slice arrives
    // last), resets the counter for the next call and writes the tile.  No
    // workgroup ever waits for another.  The partials are written and read
    // with the device-coherent cache policy (sc1, the policy hipcc itself
    // gives agent-scope atomic loads and stores on gfx950), the stores have
    // completed (s_waitcnt) before the ticket is taken, and the ticket is an
    // agent-scope atomic, so no cache-wide write-back or invalidate is
    // needed.
    if (split_tile >= 0) {
        constexpr int CPOL = 16;                           // sc1
        const int S = p.sk_split;
        constexpr int PER_WAVE = RM * RN * 64;             // 16-byte pieces per wave and slice
        const __amdgpu_buffer_rsrc_t rws =
            make_rsrc(reinterpret_cast<const char *>(p.ws) + (int64_t)split_tile * S * NW * PER_WAVE * 16);
        const uint32_t wave_off = (uint32_t)(wave * PER_WAVE + lane) * 16u;
        const uint32_t mine = (uint32_t)(slice * NW * PER_WAVE) * 16u + wave_off;
#pragma unroll
        for (int i = 0; i < RM; ++i)
#pragma unroll
            for (int j = 0; j < RN; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), rws,
                                                       mine + (uint32_t)((i * RN + j) * 64 * 16), 0, CPOL);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);                     // this wave's partial has landed
        __syncthreads();                                   // ... and every wave's
        // (the flag lives in the first LDS word: every wave's loads have
        // landed, so no direct load can still write there)
        int *sk_last = reinterpret_cast<int *>(smem);
        if (tid == 0)
            *sk_last = __hip_atomic_fetch_add(p.ws_flags + split_tile, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) == S - 1;
        __syncthreads();
        if (!*sk_last) return;
        // Sum slice by slice, CH accumulators at a time, so that CH loads are
        // in flight per wait.
        constexpr int NACC = RM * RN, CH = 8;
        static_assert(NACC % CH == 0, "accumulator chunks");
        const uint32_t sstride = (uint32_t)(NW * PER_WAVE) * 16u;
        static_for<0, NACC / CH>([&](auto chunk) {
            constexpr int c0 = decltype(chunk)::value * CH;
            f32x4 sum[CH];
#pragma unroll
            for (int c = 0; c < CH; ++c)
                sum[c] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rws, wave_off + (uint32_t)((c0 + c) * 64 * 16), 0, CPOL));
            for (int sl = 1; sl < S; ++sl) {
                f32x4 t[CH];
#pragma unroll
                for (int c = 0; c < CH; ++c)
                    t[c] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rws, sl * sstride + wave_off + (uint32_t)((c0 + c) * 64 * 16),
                                                         0, CPOL));
#pragma unroll
                for (int c = 0; c < CH; ++c) sum[c] += t[c];
            }
#pragma unroll
            for (int c = 0; c < CH; ++c) acc[(c0 + c) / RN][(c0 + c) % RN] = sum[c];
        });
        if (tid == 0) __hip_atomic_store(p.ws_flags + split_tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: fp32 -> output type, store mask of the primer's s5 ----
    // Lane l holds C[m][n] for m = 16 i + l % 16, n = 16 j + 4 (l / 16) + r.
    // The tile goes through LDS a band of whole tile rows at a time: in pass
    // p, the waves that hold rows p*PR .. p*PR + PR - 1 write them, converted
    // to the output type (round to nearest even), into LDS (row stride
    // BN*ES + 16 bytes); after a barrier every wave reads back whole tile
    // rows (16 bytes per lane, LPR lanes per row) and stores them, so each
    // store instruction writes one or more complete BN-wide rows of C.  A
    // lane whose 16 bytes lie inside N on a 4-byte aligned row stores them
    // with one 16-byte store; rows past M are never stored.  Only on an edge
    // tile (it passes N, or C's rows are not all 4-byte aligned) does a
    // second step store what the 16-byte stores left out: a chunk cut by N
    // element by element, a whole 16-bit chunk on a row that starts 2 bytes
    // past a 4-byte boundary as one element, three element pairs and one
    // element (all naturally aligned).  Chunks past N are never stored.
    constexpr int ES = (CT == OUT_F32) ? 4 : 2;
    constexpr int CE = 16 / ES;                    // elements per 16-byte chunk
    const char *Cbase = (const char *)p.C + ((int64_t)batch * p.sC + (int64_t)m0 * p.ldc + n0) * ES;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cbase);
    const int valid_n = N - n0;                    // columns of C from this tile's first one
    const bool rows_al4 = (((uintptr_t)Cbase | (uintptr_t)(p.ldc * ES)) & 3) == 0;
    const bool edge = valid_n < BN || !rows_al4;   // uniform over the workgroup
    __builtin_amdgcn_s_barrier();                  // every wave is done with the stages
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int wrow = lane & 15, wcol = 4 * (lane >> 4);
    constexpr int RS = BN * ES + 16;
    constexpr int BUDGET = STAGES * STAGE * 16;
    constexpr int PR = (WTM * RS <= BUDGET) ? WTM : (WTM / 2 * RS <= BUDGET) ? WTM / 2 : WTM / 4;
    static_assert(PR % 16 == 0 && WTM % PR == 0 && PR * RS <= BUDGET, "epilogue pass fits in LDS");
    constexpr int LPR = BN * ES / 16;                 // lanes per row
    static_assert(64 % LPR == 0, "whole rows per store instruction");
    constexpr int RPS = 64 / LPR;                     // rows per store instruction
    static_assert(PR % (NW * RPS) == 0, "rows spread evenly over the waves");
    constexpr int NST = PR / (NW * RPS);              // store instructions per wave and pass
    char *const rows = reinterpret_cast<char *>(smem);
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const int cc = (lane % LPR) * CE;                 // first column of the lane's chunk
    const bool full = cc + CE <= valid_n;
#pragma unroll
    for (int pass = 0; pass < BM / PR; ++pass) {
        constexpr int BPP = PR / 16;                  // 16-row blocks per pass
        if (wave_m == pass * PR / WTM) {
            const int i0 = (pass * PR % WTM) / 16;
#pragma unroll
            for (int ib = 0; ib < BPP; ++ib) {
#pragma unroll
                for (int j = 0; j < RN; ++j) {
                    // (i0 + ib) is uniform; select the block without
                    // dynamic indexing of the accumulator array
                    f32x4 v = acc[0][j];
#pragma unroll
                    for (int i = 1; i < RM; ++i) if (i == i0 + ib) v = acc[i][j];
                    char *dst = rows + (ib * 16 + wrow) * RS + (wave_n * WTN + 16 * j + wcol) * ES;
                    if constexpr (CT == OUT_F32) {
                        *reinterpret_cast<f32x4 *>(dst) = v;
                    } else {
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
                        *reinterpret_cast<u32x2 *>(dst) = w;
                    }
                }
            }
        }
        __syncthreads();
        u32x4 w[NST];
#pragma unroll
        for (int t = 0; t < NST; ++t) {
            const int r = (wave * NST + t) * RPS + lane / LPR;
            w[t] = *reinterpret_cast<const u32x4 *>(rows + r * RS + (lane % LPR) * 16);
        }
#pragma unroll
        for (int t = 0; t < NST; ++t) {
            const int cm = pass * PR + (wave * NST + t) * RPS + lane / LPR;
            const bool al4 = (((uintptr_t)Cbase + (uintptr_t)((int64_t)cm * p.ldc * ES)) & 3) == 0;
            const uint32_t off = (m0 + cm < M && full && al4) ? (uint32_t)(cm * p.ldc * ES + cc * ES) : OOB_OFFSET;
            __builtin_amdgcn_raw_buffer_store_b128(w[t], rc, off, 0, STORE_NT);
        }
        store_data_read_all(w);
        if (edge) {
#pragma unroll
            for (int t = 0; t < NST; ++t) {
                const int cm = pass * PR + (wave * NST + t) * RPS + lane / LPR;
                const bool al4 = (((uintptr_t)Cbase + (uintptr_t)((int64_t)cm * p.ldc * ES)) & 3) == 0;
                if (m0 + cm < M && cc < valid_n && !(full && al4)) {
                    const uint32_t row_off = (uint32_t)(cm * p.ldc + cc) * ES;
                    if constexpr (ES == 2) {
                        if (full) {
                            // 16-bit row starting 2 bytes past a 4-byte
                            // boundary: e0, (e1 e2), (e3 e4), (e5 e6), e7
                            const uint16_t e0 = (uint16_t)w[t][0], e7 = (uint16_t)(w[t][3] >> 16);
                            const uint32_t p0 = (w[t][0] >> 16) | (w[t][1] << 16);
                            const uint32_t p1 = (w[t][1] >> 16) | (w[t][2] << 16);
                            const uint32_t p2 = (w[t][2] >> 16) | (w[t][3] << 16);
                            __builtin_amdgcn_raw_buffer_store_b16(e0, rc, row_off, 0, STORE_NT);
                            __builtin_amdgcn_raw_buffer_store_b32(p0, rc, row_off + 2, 0, STORE_NT);
                            __builtin_amdgcn_raw_buffer_store_b32(p1, rc, row_off + 6, 0, STORE_NT);
                            __builtin_amdgcn_raw_buffer_store_b32(p2, rc, row_off + 10, 0, STORE_NT);
                            __builtin_amdgcn_raw_buffer_store_b16(e7, rc, row_off + 14, 0, STORE_NT);
                            store_data_read(e0);
                            store_data_read(p0);
                            store_data_read(p1);
                            store_data_read(p2);
                            store_data_read(e7);
                        } else {
#pragma unroll
                            for (int e = 0; e < CE; ++e) {
                                const uint16_t x = (uint16_t)(w[t][e / 2] >> (16 * (e % 2)));
                                const uint32_t o = cc + e < valid_n ? row_off + 2 * e : OOB_OFFSET;
                                __builtin_amdgcn_raw_buffer_store_b16(x, rc, o, 0, STORE_NT);
                                store_data_read(x);
                            }
                        }
                    } else {
                        // fp32: rows are 4-byte aligned, so only a chunk cut by N gets here
#pragma unroll
                        for (int e = 0; e < CE; ++e) {
                            const uint32_t x = w[t][e];
                            const uint32_t o = cc + e < valid_n ? row_off + 4 * e : OOB_OFFSET;
                            __builtin_amdgcn_raw_buffer_store_b32(x, rc, o, 0, STORE_NT);
                            store_data_read(x);
                        }
                    }
                }
            }
        }
        if (pass + 1 < BM / PR) __syncthreads();      // the rows are rewritten by the next pass
    }
}

}  // namespace tdg
