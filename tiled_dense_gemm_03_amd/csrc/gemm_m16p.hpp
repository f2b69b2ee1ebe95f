// gemm_m16p.hpp -- persistent form of the 16x16x32 MFMA kernel.
//
// Same operand path as gemm_m16_kernel (direct global -> LDS loads, the
// XOR-swizzled LDS layouts, 16x16x32 MFMAs issued as mfma(B, A), one loop
// body per K tile with the refill of the freed stage spread between the
// last K step's MFMAs), with two differences:
//
//  * One workgroup per CU that walks its output tiles in turn (tile w,
//    w + G, w + 2G, ... of the XCD-aware order, G workgroups).  The K loop
//    runs over the concatenation of those tiles' K ranges, so the loads
//    running STAGES K tiles ahead cross into the next output tile: its
//    first operand tiles arrive while the current tile's last MFMAs run,
//    and no tile after the first waits for the full load latency.
//  * The epilogue runs between two K iterations, while the stages already
//    hold the next tile's operands, so it goes through a small staging area
//    of its own (per wave, 16 rows of 16-bit values; for fp32, 16 rows of
//    each wave row as whole tile rows); the stores of one tile drain while
//    the next tile computes.
//
// The NineToothed primer's decomposition (s4: one program per output tile,
// K as a loop in the program) is unchanged: a workgroup runs several
// programs one after another.  No split-K here.
#pragma once

#include "gemm_m16.hpp"

namespace tdg {

template <int BM, int BN, int WM, int WN, int STAGES, bool TRANSA, bool TRANSB, int AB, int CT>
__global__ __launch_bounds__(WM * WN * 64) void gemm_m16p_kernel(GemmArgs p) {
    constexpr int BK = 64, KS = 2, KG = 8, BNG = BN / GRAN, BMG = BM / GRAN;
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
    static_assert((STAGES - 1) * NDMA < 64, "vmcnt range");
    static_assert(STAGE * 16 * STAGES <= 160 * 1024, "LDS budget");
    constexpr int RPB = 64 / BNG, RPA = 64 / BMG;
    constexpr int NVB = TRANSB ? 1 : 16 / ((NW * RPB) % 16 == 0 ? 16 : ((NW * RPB) % 8 == 0 ? 8 : ((NW * RPB) % 4 == 0 ? 4 : ((NW * RPB) % 2 == 0 ? 2 : 1))));
    constexpr int NVA = !TRANSA ? 1 : 16 / ((NW * RPA) % 16 == 0 ? 16 : ((NW * RPA) % 8 == 0 ? 8 : ((NW * RPA) % 4 == 0 ? 4 : ((NW * RPA) % 2 == 0 ? 2 : 1))));

    // A staging area outside the stages (which hold the next tile's
    // operands when the epilogue runs).  16-bit output: per wave, one 16-row
    // block of its sub-tile.  fp32 output: one 16-row block of every wave
    // row, held as whole tile rows (WM x 16 rows of BN * 4 bytes, 16-byte
    // chunks XOR-swizzled by the row so neither the writes nor the reads
    // conflict; no padding, so 2 x 16 rows of 1 KiB fill what two 64 KiB
    // stages leave of the LDS).
    constexpr int ES = (CT == OUT_F32) ? 4 : 2;
    constexpr int SROW = WTN * ES + 16;                      // staged row (16-bit), padded by 16 bytes
    constexpr int SR = 16;                                   // rows staged at a time (16-bit)
    constexpr int RB = BN * 4;                               // bytes of a tile row (fp32)
    constexpr int CPR32 = RB / 16;                           // 16-byte chunks of a tile row (fp32)
    static_assert(CT != OUT_F32 || (CPR32 >= 16 && (CPR32 & (CPR32 - 1)) == 0 && 64 % CPR32 == 0),
                  "fp32 tile rows: a power of two of 16..64 chunks");
    constexpr int STG = (CT == OUT_F32) ? WM * 16 * CPR32 : NW * SR * SROW / 16;
    static_assert((STAGE * STAGES + STG) * 16 <= 160 * 1024, "LDS budget");
    __shared__ u32x4 smem[STAGES * STAGE + STG];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave / WN, wave_n = wave % WN;
    const int M = p.M, N = p.N, K = p.K;
    const int64_t lda = p.lda, ldb = p.ldb;
    const int nk = (K + BK - 1) / BK;               // >= 1: the host launches this kernel with K > 0 only
    const int total = p.dp_tiles;                   // output tiles of the whole call
    const int G = gridDim.x;
    const int w0 = xcd_order(blockIdx.x, G);        // this workgroup's first tile; then + G, + 2G, ...
    const int ntile = w0 < total ? (total - w0 + G - 1) / G : 0;
    const int nsteps = ntile * nk;

    // ---- per-lane load offsets that do not depend on the tile ----
    const int kc_row = wave * 8 + (lane >> 3);
    const int kc_g = (lane & 7) ^ kx16(kc_row);
    const uint32_t a_kc = (uint32_t)((kc_row * lda + kc_g * GRAN) * 2);
    const uint32_t b_kc = (uint32_t)((kc_row * ldb + kc_g * GRAN) * 2);
    const uint32_t a_qs = TRANSA ? (uint32_t)(NW * RPA * lda * 2) : (uint32_t)(NW * 8 * lda * 2);
    const uint32_t b_qs = TRANSB ? (uint32_t)(NW * 8 * ldb * 2) : (uint32_t)(NW * RPB * ldb * 2);

    // ---- the tile the loads are working on ("pf": STAGES K tiles ahead of
    // the MFMAs) ----
    int pf_r = 0, pf_kt = 0;                        // round (tile w0 + r*G) and K tile
    int pf_m0 = 0, pf_n0 = 0, pf_arows = 0, pf_brows = 0;
    const uint16_t *pf_A = p.A, *pf_B = p.B;
    uint32_t a_lane[NVA], b_lane[NVB];
    auto pf_tile = [&]() {
        // a tile past this workgroup's last one loads nothing (no valid rows,
        // no valid columns)
        const bool live = pf_r < ntile;
        int batch = 0, tm = 0, tn = 0;
        if (live) tile_of(p, w0 + pf_r * G, batch, tm, tn);
        pf_m0 = live ? tm * BM : M;
        pf_n0 = live ? tn * BN : N;
        pf_arows = M - pf_m0 < BM ? M - pf_m0 : BM;
        pf_brows = N - pf_n0 < BN ? N - pf_n0 : BN;
        pf_A = TRANSA ? p.A + (int64_t)batch * p.sA + pf_m0 : p.A + (int64_t)batch * p.sA + (int64_t)pf_m0 * lda;
        pf_B = TRANSB ? p.B + (int64_t)batch * p.sB + (int64_t)pf_n0 * ldb : p.B + (int64_t)batch * p.sB + pf_n0;
        if constexpr (!TRANSA) {
            a_lane[0] = a_kc;
        } else {
#pragma unroll
            for (int v = 0; v < NVA; ++v) {
                const int kr = RPA * wave + lane / BMG;
                const int k = RPA * (v * NW) + kr;
                const int c = (lane % BMG) ^ nx16(k);
                a_lane[v] = (pf_m0 + c * GRAN < M) ? (uint32_t)((kr * lda + c * GRAN) * 2) : OOB_OFFSET;
            }
        }
        if constexpr (TRANSB) {
            b_lane[0] = b_kc;
        } else {
#pragma unroll
            for (int v = 0; v < NVB; ++v) {
                const int kr = RPB * wave + lane / BNG;
                const int k = RPB * (v * NW) + kr;
                const int c = (lane % BNG) ^ nx16(k);
                b_lane[v] = (pf_n0 + c * GRAN < N) ? (uint32_t)((kr * ldb + c * GRAN) * 2) : OOB_OFFSET;
            }
        }
    };
    pf_tile();
    auto pf_advance = [&]() {
        if (++pf_kt == nk) {
            pf_kt = 0;
            ++pf_r;
            pf_tile();
        }
    };
    const int kc_klim = K - kc_g * GRAN;

    auto dma_op = [&](auto qtag, u32x4 *sa) {
        constexpr int q = decltype(qtag)::value;
        const int k0 = pf_kt * BK;
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr_of(sa) + (uint32_t)wave * 1024u);
        if constexpr (q < QA) {
            if constexpr (!TRANSA) {
                const u32x4 rs = rsrc_words_n(pf_A + k0, records_of((int64_t)(pf_arows - 1) * lda + K - k0));
                const uint32_t off = (k0 < kc_klim ? a_lane[0] : OOB_OFFSET) + (uint32_t)q * a_qs;
                dma16<(uint32_t)(q * NW) * 1024u>(rs, off, base);
            } else {
                const u32x4 rs = rsrc_words_n(pf_A + (int64_t)k0 * lda,
                                              records_of((int64_t)(K - k0 - 1) * lda + (M - pf_m0)));
                const uint32_t off = a_lane[q % NVA] + (uint32_t)q * a_qs;
                dma16<(uint32_t)(q * NW) * 1024u>(rs, off, base);
            }
        } else {
            constexpr int qb = q - QA;
            if constexpr (TRANSB) {
                const u32x4 rs = rsrc_words_n(pf_B + k0, records_of((int64_t)(pf_brows - 1) * ldb + K - k0));
                const uint32_t off = (k0 < kc_klim ? b_lane[0] : OOB_OFFSET) + (uint32_t)qb * b_qs;
                dma16<(uint32_t)(A_SLOTS * 16 + qb * NW * 1024)>(rs, off, base);
            } else {
                const u32x4 rs = rsrc_words_n(pf_B + (int64_t)k0 * ldb,
                                              records_of((int64_t)(K - k0 - 1) * ldb + (N - pf_n0)));
                const uint32_t off = b_lane[qb % NVB] + (uint32_t)qb * b_qs;
                dma16<(uint32_t)(A_SLOTS * 16 + qb * NW * 1024)>(rs, off, base);
            }
        }
    };

    // ---- fragment addresses (as in gemm_m16_kernel) ----
    const int fr = lane & 15, fg = lane >> 4;
    int a_b[KS], bt_b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        a_b[ks] = (wave_m * WTM + fr) * KG + ((4 * ks + fg) ^ ((lane >> 1) & 7));
        bt_b[ks] = (wave_n * WTN + fr) * KG + ((4 * ks + fg) ^ ((lane >> 1) & 7));
    }
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
    auto tr_read = [&](const u32x4 *st, int byte_off, u32x4 &frag, auto htag) {
        constexpr int h = decltype(htag)::value;
        const char *base = reinterpret_cast<const char *>(st);
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(base + byte_off));
        const uint64_t w = __builtin_bit_cast(uint64_t, v);
        frag[2 * h] = (uint32_t)w;
        frag[2 * h + 1] = (uint32_t)(w >> 32);
    };
    constexpr int DA = TRANSA ? 2 * RM : RM;
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
        for (int j = 0; j < RN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // ---- epilogue of one output tile, from the accumulators ----
    // Lane l holds C[m][n .. n+3] for m = 16 i + l % 16, n = 16 j + 4 (l / 16)
    // of the wave's sub-tile.  Interior tiles: each 16-row block (fp32:
    // each half block) is converted (round to nearest even) into the wave's
    // staging area and read back as 16-byte row pieces, so each store
    // instruction writes whole row segments.  A ragged right edge or an
    // unaligned C takes element stores.  Rows past M are never stored.
    // Each store address is a per-lane offset plus a uniform one, so the
    // epilogue keeps almost nothing live across the K loop.
    const bool c_aligned = (((uintptr_t)p.C | (uintptr_t)(p.ldc * ES) | (uintptr_t)(p.sC * ES)) & 3) == 0;
    const uint32_t lane_off = (uint32_t)(fr * p.ldc + 4 * fg) * ES;
    char *const stage_r = reinterpret_cast<char *>(smem + STAGES * STAGE) + wave * SR * SROW;
    char *const stage_w = stage_r + (fr % SR) * SROW;
    auto epilogue = [&](int r) {
        int batch, tm, tn;
        tile_of(p, w0 + r * G, batch, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const char *Cbase = (const char *)p.C + ((int64_t)batch * p.sC + (int64_t)(m0 + wave_m * WTM) * p.ldc +
                                                 n0 + wave_n * WTN) * ES;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cbase);
        const __amdgpu_buffer_rsrc_t rc_tile =
            make_rsrc((const char *)p.C + ((int64_t)batch * p.sC + (int64_t)m0 * p.ldc + n0) * ES);
        const bool vec_store = (n0 + BN <= N) && c_aligned;
        const int cols_left = N - n0 - wave_n * WTN - 4 * fg;      // valid columns from the lane's first one
#pragma unroll
        for (int i = 0; i < RM; ++i) {
            const int rows_left = M - m0 - wave_m * WTM - 16 * i;    // uniform
            const uint32_t vo = fr < rows_left ? lane_off : OOB_OFFSET;
            const uint32_t so_row = (uint32_t)(16 * i * p.ldc) * ES;
#pragma unroll
            for (int j = 0; j < RN; ++j) {
                const uint32_t so = so_row + (uint32_t)(16 * j * ES);
                const f32x4 v = acc[i][j];
                if (vec_store) {
                    if constexpr (CT == OUT_F32) {
                        // staged below, half a block at a time
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
                        *reinterpret_cast<u32x2 *>(stage_w + (16 * j + 4 * fg) * 2) = w;
                        store_data_read(w);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t voe = (16 * j + e < cols_left) ? vo + (uint32_t)(e * ES) : OOB_OFFSET;
                        if constexpr (CT == OUT_F32) {
                            // (the words of the whole vector: hipcc's bit cast of a
                            // single vector element reads element 0 whatever the index)
                            const uint32_t x = __builtin_bit_cast(u32x4, v)[e];
                            __builtin_amdgcn_raw_buffer_store_b32(x, rc, voe, so, STORE_NT);
                            store_data_read(x);
                        } else if constexpr (CT == OUT_F16) {
                            const uint16_t x = __builtin_bit_cast(uint16_t, (_Float16)v[e]);
                            __builtin_amdgcn_raw_buffer_store_b16(x, rc, voe, so, STORE_NT);
                            store_data_read(x);
                        } else {
                            const uint16_t x = __builtin_bit_cast(uint16_t, (__bf16)v[e]);
                            __builtin_amdgcn_raw_buffer_store_b16(x, rc, voe, so, STORE_NT);
                            store_data_read(x);
                        }
                    }
                }
                if (CT != OUT_F32 || !vec_store) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            if constexpr (CT == OUT_F32) {
                // block i of every wave row at once (vec_store is uniform over
                // the workgroup): staged row R = wave_m * 16 + fr holds tile row
                // wave_m * WTM + 16 i + fr; each wave then stores whole tile
                // rows, RPI rows of CPR32 chunks per instruction.
                constexpr int RPI = 64 / CPR32, PRW = WM * 16, NT = PRW / (NW * RPI);
                static_assert(NT * NW * RPI == PRW, "staged rows spread evenly over the waves");
                if (vec_store) {
                    char *const stg = reinterpret_cast<char *>(smem + STAGES * STAGE);
                    if (i > 0) __syncthreads();                  // block i - 1 has been read back
                    const int R = wave_m * 16 + fr;
#pragma unroll
                    for (int j = 0; j < RN; ++j) {
                        const int c = (wave_n * WTN + 16 * j + 4 * fg) / 4;
                        *reinterpret_cast<f32x4 *>(stg + R * RB + ((c ^ (R & 15)) * 16)) = acc[i][j];
                    }
                    __syncthreads();
                    u32x4 w[NT];
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const int Rr = (wave * NT + t) * RPI + lane / CPR32, c = lane % CPR32;
                        w[t] = *reinterpret_cast<const u32x4 *>(stg + Rr * RB + ((c ^ (Rr & 15)) * 16));
                    }
                    static_assert(RPI == 1, "one tile row per store instruction");
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        // the row is uniform over the wave: its offset goes in
                        // the scalar operand and the row test is a branch, so
                        // only the lane's 16-byte column offset is per lane
                        // (per-lane row offsets hoisted out of the tile walk
                        // would not fit in the register file)
                        const int Rr = wave * NT + t;
                        const int row = (Rr / 16) * WTM + 16 * i + Rr % 16;     // row of the tile
                        if (m0 + row < M)
                            __builtin_amdgcn_raw_buffer_store_b128(w[t], rc_tile, (uint32_t)lane * 16u,
                                                                   (int)((int64_t)row * p.ldc * ES), STORE_NT);
                    }
                    store_data_read_all(w);
#pragma unroll
                    for (int j = 0; j < RN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
            } else {
                // read back the 16 staged rows: 16-byte pieces, rows of the
                // block t * RPI + lane / CPR, piece lane % CPR
                constexpr int CPR = WTN * 2 / 16, RPI = 64 / CPR;
                static_assert(CPR * RPI == 64 && 16 % RPI == 0, "row pieces must tile a wave");
                if (vec_store) {
#pragma unroll
                    for (int t = 0; t < 16 / RPI; ++t) {
                        const int row = t * RPI + lane / CPR, piece = lane % CPR;
                        const u32x4 w = *reinterpret_cast<const u32x4 *>(stage_r + row * SROW + piece * 16);
                        const uint32_t off = row < rows_left ? (uint32_t)(row * p.ldc + piece * 8) * ES : OOB_OFFSET;
                        __builtin_amdgcn_raw_buffer_store_b128(w, rc, off, so_row, STORE_NT);
                        store_data_read(w);
                    }
                }
            }
        }
    };

    u32x4 af[2][RM], bf[2][RN];

    if (nsteps > 0) {
        static_for<0, STAGES>([&](auto s) {
            static_for<0, NDMA>([&](auto q) { dma_op(q, smem + decltype(s)::value * STAGE); });
            pf_advance();
        });
        wait_vm_lgkm0<(STAGES - 1) * NDMA>();
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        frags_from(smem, 0, af[0], bf[0]);
    }

    // One K tile per iteration (the 16x16x32 kernel's loop body); the loads
    // of the refill belong to whatever tile is STAGES K tiles ahead.  After
    // the last K tile of an output tile, its epilogue; the next iteration's
    // MFMAs start the following tile on zeroed accumulators.
    int s_cur = 0, kt = 0, r = 0;
    for (int step = 0; step < nsteps; ++step) {
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
        constexpr int NSUB = NDMA;
        static_for<0, NSUB>([&](auto sub) {
            constexpr int s0 = decltype(sub)::value;
            static_for<s0 * NMF / NSUB, (s0 + 1) * NMF / NSUB>([&](auto m) {
                constexpr int i = decltype(m)::value / RN, j = decltype(m)::value % RN;
                acc[i][j] = mfma_16x16x32<AB>(bf[1][j], af[1][i], acc[i][j]);
            });
            static_for<s0 * NDS / NSUB, (s0 + 1) * NDS / NSUB>([&](auto d) { frag_op(d, nxt, 0, af[0], bf[0]); });
            dma_op(sub, cur);
            __builtin_amdgcn_sched_barrier(0);
        });
        pf_advance();
        if (++kt == nk) {
            epilogue(r);
            kt = 0;
            ++r;
        }
        s_cur = s_nxt;
    }
    __builtin_amdgcn_s_waitcnt(0);
}

}  // namespace tdg
