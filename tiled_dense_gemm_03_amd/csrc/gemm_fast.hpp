// gemm_fast.hpp -- the vectorised MFMA GEMM kernel for gfx950 (aligned operands).
//
// Same decomposition as the general kernel (one workgroup per output tile,
// K loop inside the workgroup, fp32 accumulators; NineToothed GEMM primer s4),
// built on three gfx950 features:
//
//  * Direct global -> LDS loads in buffer form (buffer_load_dwordx4 ... lds).
//    Lane l of an instruction writes its 16 bytes at LDS base + 16*l, so the
//    LDS layout is produced by choosing, for each LDS slot, which global
//    granule its lane fetches.  A lane whose slot is padding or whose element
//    lies outside the matrix uses an offset past the buffer's range: the
//    hardware skips the memory access and writes zeros, which is exactly the
//    zero-filled masked read of the primer's s5, with no branch and no staging
//    registers.
//  * v_mfma_f32_32x32x16_{f16,bf16} with fp32 accumulators.
//  * ds_read_b64_tr_b16 for the B operand of NN products: B stays N-contiguous
//    in LDS (as it is in memory) and the transposing LDS read delivers the
//    K-runs the MFMA B operand wants.  Within each 16-lane group, result lane
//    4q+p receives element p of the 8-byte rows supplied by lanes q, 4+q,
//    8+q and 12+q; with lanes 4j..4j+3 pointing at 16 consecutive columns of
//    K row j, lane i receives column i of rows 0..3.
//
// LDS layouts (16-byte granules of 8 elements; STAGES copies):
//   A, and B of TN:  [rows][BK/8 granules], K-contiguous.  Granule g of row r
//                    sits at position g ^ ((r ^ (r >> 3)) & 7) for BK = 64 and
//                    g ^ ((r >> 2) & 3) for BK = 32.
//   B of NN:         [BK k][BN/8 granules], N-contiguous; granule c of row k
//                    at position c ^ (4 * (k & 3)).
// Each XOR puts the 16 granules that 16 neighbouring lanes read at once on 16
// distinct 16-byte bank groups (the LDS has 64 four-byte banks), so operand
// reads are conflict-free, while every stage stays a whole number of 1 KiB
// direct-load runs with no padding.  The XOR terms are such that each
// operand needs only a few base addresses per lane (the rest are
// compile-time offsets).  Writer and reader derive positions from the same
// formulas (the Croqtile tutorial ch.4 notes that a swizzled store and the
// operand load must agree on the swizzle).
//
// Pipeline: the STAGES LDS stages are separate objects.  Loads run STAGES-1
// tiles ahead; the fragments of K step kk+1 are read while the MFMAs of step
// kk run; the single barrier per K tile sits before the tile's last step,
// whose fragments are already in registers, and the refill of the freed stage
// is spread between that step's MFMAs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.hpp"
#include "gemm_kernel.hpp"

namespace tdg {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t OOB_OFFSET = 0x80000000u;    // >= num_records: load returns zeros
constexpr int32_t BUF_RECORDS = 0x7fffffff;     // every valid offset is below 2^31
constexpr int32_t BUF_FLAGS = 0x00020000;       // raw 32-bit buffer (gfx9 word 3)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, BUF_RECORDS, BUF_FLAGS);
}

// The same buffer descriptor as four dwords (base, stride 0, records, flags).
__device__ __forceinline__ u32x4 rsrc_words(const void *base) {
    const uint64_t a = (uint64_t)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    r[2] = (uint32_t)BUF_RECORDS;
    r[3] = (uint32_t)BUF_FLAGS;
    return r;
}

// One direct global -> LDS load of 16 bytes per lane: lane l's granule at
// byte offset voff of the buffer lands at LDS address lds_addr + 16*l
// (zeros for an out-of-range offset).  Written as inline assembly so that
// the compiler's automatic wait insertion, which cannot tell one LDS stage
// from another here, does not add a wait for these loads before every LDS
// read; the kernel waits for them explicitly (vmcnt) before its barriers.
// M0 (which holds the LDS address) is saved and restored around the load.
// The LDS address is lds_base + IMM (IMM a compile-time byte offset), so a
// whole stage needs a single address register.
template <uint32_t IMM>
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t voff, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_add_u32 m0, %3, %4\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"(lds_base), "n"(IMM)
        : "memory", "scc");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// s_waitcnt immediate (gfx9 encoding): wait until at most VM vector memory
// operations are outstanding and every LDS operation has completed.
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
}

// Order the instructions of one compute block: MF MFMAs with DS LDS reads
// spread between them, PER MFMAs before each read (a scheduling constraint
// only; it changes no result).
template <int MF, int DS, int PER>
__device__ __forceinline__ void interleave_rec() {
    if constexpr (MF > 0 || DS > 0) {
        constexpr int take = MF < PER ? MF : PER;
        if constexpr (take > 0) __builtin_amdgcn_sched_group_barrier(0x008, take, 0);
        if constexpr (DS > 0) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            interleave_rec<MF - take, DS - 1, PER>();
        } else {
            interleave_rec<MF - take, 0, PER>();
        }
    }
}

template <int NMF, int NDS>
__device__ __forceinline__ void interleave_hint() {
    constexpr int PER = NDS > 0 ? (NMF > NDS ? NMF / NDS : 1) : NMF;
    interleave_rec<NMF, NDS, PER>();
}

// Compile-time loop: f(std::integral_constant<int, i>) for i in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Position of granule g of row r in a K-contiguous tile with rows of BK.
template <int BK>
__device__ __forceinline__ int kpos(int r, int g) {
    if constexpr (BK == 64) return r * 8 + (g ^ ((r ^ (r >> 3)) & 7));
    else return r * 4 + (g ^ ((r >> 2) & 3));
}

// Position of granule c of row k in an N-contiguous NN B tile (BNG granules per row).
template <int BNG>
__device__ __forceinline__ int npos(int k, int c) { return k * BNG + (c ^ (4 * (k & 3))); }

// Tile geometry.
template <int BM, int BN, int BK, int STAGES, bool TRANSB>
struct FastGeom {
    static constexpr int KG = BK / GRAN;                        // granules per K-contiguous row
    static constexpr int BNG = BN / GRAN;                       // granules per NN B row
    static constexpr int A_SLOTS = BM * KG;
    static constexpr int B_SLOTS = BN * KG;                     // BK x BN either way
    static constexpr int STAGE = A_SLOTS + B_SLOTS;             // granules per stage
    // Direct loads are issued in whole-wave instructions; when a stage is not
    // a multiple of one instruction per wave, the spare instructions write
    // zeros into a 1 KiB scratch area so that every wave issues the same count.
    template <int NW>
    static constexpr bool needs_trash() { return (A_SLOTS / 64) % NW != 0 || (B_SLOTS / 64) % NW != 0; }
    template <int NW>
    static constexpr int lds_bytes() { return STAGE * 16 * STAGES + (needs_trash<NW>() ? 1024 : 0); }
};

template <int BM, int BN, int WM, int WN, int BK, int STAGES, bool TRANSB, int AB, int CT>
__global__ __launch_bounds__(WM * WN * 64) void gemm_fast_kernel(GemmArgs p) {
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int RM = WTM / 32, RN = WTN / 32;
    static_assert(RM * 32 == WTM && RN * 32 == WTN, "wave tile must be a multiple of 32");
    static_assert(BK == 32 || BK == 64, "BK is 32 or 64");
    static_assert(STAGES >= 2 && STAGES <= 5, "2 to 5 stages");
    using G = FastGeom<BM, BN, BK, STAGES, TRANSB>;
    constexpr int KS = BK / 16;                      // MFMA K steps per tile
    constexpr int KG = G::KG, BNG = G::BNG;
    constexpr int A_SLOTS = G::A_SLOTS, B_SLOTS = G::B_SLOTS, STAGE = G::STAGE;
    static_assert(G::template lds_bytes<NW>() <= 160 * 1024, "LDS budget");
    static_assert(TRANSB || BNG >= 16, "NN B rows of at least 16 granules");
    static_assert(RM == 1 || WTM % 64 == 0, "A fragment bases assume 64-row wave tiles");
    static_assert(!TRANSB || RN == 1 || WTN % 64 == 0, "B fragment bases assume 64-row wave tiles");
    constexpr int NIA = A_SLOTS / 64, NIB = B_SLOTS / 64;     // wave-wide load instructions per stage
    static_assert(NIA * 64 == A_SLOTS && NIB * 64 == B_SLOTS, "stage must be whole 1 KiB runs");
    constexpr int QA = (NIA + NW - 1) / NW, QB = (NIB + NW - 1) / NW;   // per wave (the last may be idle)
    constexpr int NDMA = QA + QB;
    static_assert((STAGES - 1) * NDMA < 64, "vmcnt range");

    // Stages back to back, then the 1 KiB scratch area for spare loads.  After
    // the K loop the same memory stages the output tile (epilogue).
    __shared__ u32x4 smem[STAGES * STAGE + (G::template needs_trash<NW>() ? 64 : 0)];
    u32x4 *const trash = smem + STAGES * STAGE;
    auto stage_ptr = [&](auto tag) -> u32x4 * { return smem + decltype(tag)::value * STAGE; };

    int batch, tm, tn;
    tile_coords(p, batch, tm, tn);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave / WN, wave_n = wave % WN;
    const int M = p.M, N = p.N, K = p.K;
    const int m0 = tm * BM, n0 = tn * BN;

    const uint16_t *Atile = p.A + (int64_t)batch * p.sA + (int64_t)m0 * p.lda;
    const uint16_t *Btile = TRANSB ? p.B + (int64_t)batch * p.sB + (int64_t)n0 * p.ldb
                                   : p.B + (int64_t)batch * p.sB + n0;

    // ---- per-lane direct-load descriptors, fixed over the K loop ----
    // Load instruction t = wave + NW*q writes LDS slots 64t .. 64t+63 of the
    // stage; the lane fetches the global granule that the layout puts in its
    // slot (the XOR swizzles are involutions), or, if that granule's row lies
    // outside the matrix, uses the out-of-range offset.  klim: the granule is
    // loaded while k0 < klim.
    uint32_t a_off[QA];
    int a_klim[QA];
#pragma unroll
    for (int q = 0; q < QA; ++q) {
        const int slot = (q * NW + wave) * 64 + lane;
        const int row = slot / KG;
        const int g = kpos<BK>(row, slot % KG) - row * KG;
        const bool ok = m0 + row < M;
        a_off[q] = ok ? (uint32_t)(row * p.lda + g * GRAN) * 2u : OOB_OFFSET;
        a_klim[q] = ok ? K - g * GRAN : -1;
    }
    uint32_t b_off[QB];
    int b_klim[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
        const int slot = (q * NW + wave) * 64 + lane;
        if constexpr (TRANSB) {
            const int row = slot / KG;
            const int g = kpos<BK>(row, slot % KG) - row * KG;
            const bool ok = n0 + row < N;
            b_off[q] = ok ? (uint32_t)(row * p.ldb + g * GRAN) * 2u : OOB_OFFSET;
            b_klim[q] = ok ? K - g * GRAN : -1;
        } else {
            const int k = slot / BNG;
            const int c = npos<BNG>(k, slot % BNG) - k * BNG;
            const bool ok = n0 + c * GRAN < N;
            b_off[q] = ok ? (uint32_t)(k * p.ldb + c * GRAN) * 2u : OOB_OFFSET;
            b_klim[q] = ok ? K - k : -1;
        }
    }

    // Direct load number q (0 <= q < NDMA) of this wave for K tile kt into
    // the stage at sa.  Every wave issues NDMA loads per tile (spare ones go
    // to the scratch area with an out-of-range offset), so one vmcnt value
    // fits all waves.
    auto dma_op = [&](auto qtag, int kt, u32x4 *sa) {
        constexpr int q = decltype(qtag)::value;
        const int k0 = kt * BK;
        // wave-relative base of this stage; spare loads go to the scratch
        // area (whose offset from the stage is fixed at link time, so it is
        // folded into the same base)
        const uint32_t base = lds_addr_of(sa) + (uint32_t)wave * 1024u;
        if constexpr (q < QA) {
            const bool live = NIA % NW == 0 || q * NW + wave < NIA;
            const uint32_t off = (live && k0 < a_klim[q]) ? a_off[q] : OOB_OFFSET;
            const uint32_t dst = live ? base : lds_addr_of(trash) - (uint32_t)(q * NW) * 1024u;
            dma16<(uint32_t)(q * NW) * 1024u>(rsrc_words(Atile + k0), off, dst);
        } else {
            constexpr int qb = q - QA;
            const bool live = NIB % NW == 0 || qb * NW + wave < NIB;
            const uint32_t off = (live && k0 < b_klim[qb]) ? b_off[qb] : OOB_OFFSET;
            const uint32_t dst = live ? base : lds_addr_of(trash) - (uint32_t)(A_SLOTS * 16 + qb * NW * 1024);
            dma16<(uint32_t)(A_SLOTS * 16 + qb * NW * 1024)>(
                rsrc_words(TRANSB ? Btile + k0 : Btile + (int64_t)k0 * p.ldb), off, dst);
        }
    };
    auto issue_to = [&](int kt, u32x4 *sa) { static_for<0, NDMA>([&](auto q) { dma_op(q, kt, sa); }); };

    // ---- fragment addresses: a few bases per lane plus constant offsets ----
    // A (and TN B) fragment i at K step kk: granule 2 kk + frag_g of row
    // wave_x * WT + 32 i + frag_row.  Rows 64 apart share the XOR term, so
    // fragment i uses base i % 2 plus 32 * (i - i % 2) rows.
    const int frag_row = lane & 31;
    const int frag_g = lane >> 5;
    int a_b[2][KS], bt_b[2][KS];
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            a_b[v][kk] = kpos<BK>(wave_m * WTM + 32 * v + frag_row, 2 * kk + frag_g);
            bt_b[v][kk] = kpos<BK>(wave_n * WTN + 32 * v + frag_row, 2 * kk + frag_g);
        }
    // NN B: byte address of the 8-byte piece lane `lane` supplies to tr read h
    // of column block j at K step kk: row 16 kk + 8 (grp >> 1) + 4 h + jr,
    // columns wave_n * WTN + 32 j + 16 (grp & 1) + 4 q4 .. +3.  The XOR term
    // depends on the row only through jr, so (kk, h) are constant offsets.
    const int grp = lane >> 4, jr = (lane & 15) >> 2, q4 = lane & 3;
    int bn_b[RN];
#pragma unroll
    for (int j = 0; j < RN; ++j) {
        const int n = wave_n * WTN + 32 * j + 16 * (grp & 1) + 4 * q4;
        bn_b[j] = npos<BNG>(8 * (grp >> 1) + jr, n / GRAN) * 16 + ((n % GRAN) / 4) * 8;
    }

    // LDS read number d (0 <= d < NDS) of K step kk's fragments.
    auto frag_op = [&](auto dtag, const u32x4 *sa, int kk, u32x4 (&af)[RM], u32x4 (&bf)[RN]) {
        constexpr int d = decltype(dtag)::value;
        const u32x4 *sb = sa + A_SLOTS;
        if constexpr (d < RM) {
            af[d] = sa[a_b[d & 1][kk] + (d & ~1) * 32 * KG];
        } else if constexpr (TRANSB) {
            constexpr int j = d - RM;
            bf[j] = sb[bt_b[j & 1][kk] + (j & ~1) * 32 * KG];
        } else {
            constexpr int j = (d - RM) / 2, h = (d - RM) % 2;
            const char *base = reinterpret_cast<const char *>(sb);
            const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(base + bn_b[j] + (16 * kk + 4 * h) * BNG * 16));
            const uint64_t w = __builtin_bit_cast(uint64_t, v);
            bf[j][2 * h] = (uint32_t)w;
            bf[j][2 * h + 1] = (uint32_t)(w >> 32);
        }
    };
    constexpr int NDS = RM + (TRANSB ? RN : 2 * RN);   // LDS reads per K step
    constexpr int NMF = RM * RN;                       // MFMAs per K step
    auto frags_from = [&](const u32x4 *sa, int kk, u32x4 (&af)[RM], u32x4 (&bf)[RN]) {
        static_for<0, NDS>([&](auto d) { frag_op(d, sa, kk, af, bf); });
    };

    f32x16 acc[RM][RN];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (K + BK - 1) / BK;
    u32x4 af[2][RM], bf[2][RN];

    // Loads of tiles past the last one are all out of range: they fetch
    // nothing and only write zeros into a stage that is never read again.
    if (nk > 0) {
        static_for<0, STAGES>([&](auto s) { issue_to(decltype(s)::value, stage_ptr(s)); });
        wait_vm_lgkm0<(STAGES - 1) * NDMA>();    // tile 0 has landed (this lane)
        __builtin_amdgcn_s_barrier();             // ... for every lane
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        frags_from(smem, 0, af[0], bf[0]);
    }

    // One K tile held in stage S (a compile-time constant).
    auto tile_iter = [&](auto stage_tag, int kt) {
        constexpr int S = decltype(stage_tag)::value;
        u32x4 *cur = stage_ptr(std::integral_constant<int, S>{});
        u32x4 *nxt = stage_ptr(std::integral_constant<int, (S + 1) % STAGES>{});
#pragma unroll
        for (int kk = 0; kk < KS - 1; ++kk) {
            frags_from(cur, kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
#pragma unroll
            for (int i = 0; i < RM; ++i)
#pragma unroll
                for (int j = 0; j < RN; ++j)
                    acc[i][j] = mfma_32x32x16<AB>(bf[kk & 1][j], af[kk & 1][i], acc[i][j]);
            interleave_hint<NMF, NDS>();
        }
        // Tile kt+1 has landed (tiles kt+2 .. kt+STAGES-1 may still be in
        // flight) and this lane's reads of stage S are done; after the
        // barrier the same holds for every lane, so stage S may be refilled.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        wait_vm_lgkm0<(STAGES - 2) * NDMA>();
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        // Last K step of the tile: its MFMAs, the next tile's first
        // fragments and the refill of stage S, spread evenly in NSUB slices
        // (each slice: some MFMAs, some LDS reads, one direct load).
        constexpr int NSUB = NDMA;
        static_for<0, NSUB>([&](auto sub) {
            constexpr int s0 = decltype(sub)::value;
            static_for<s0 * NMF / NSUB, (s0 + 1) * NMF / NSUB>([&](auto m) {
                constexpr int i = decltype(m)::value / RN, j = decltype(m)::value % RN;
                acc[i][j] = mfma_32x32x16<AB>(bf[(KS - 1) & 1][j], af[(KS - 1) & 1][i], acc[i][j]);
            });
            static_for<s0 * NDS / NSUB, (s0 + 1) * NDS / NSUB>([&](auto d) {
                frag_op(d, nxt, 0, af[KS & 1], bf[KS & 1]);
            });
            dma_op(sub, kt + STAGES, cur);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    for (int kt = 0; kt < nk; kt += STAGES) {
        static_for<0, STAGES>([&](auto s) {
            constexpr int S = decltype(s)::value;
            if (S == 0 || kt + S < nk) tile_iter(s, kt + S);
        });
    }
    __builtin_amdgcn_s_waitcnt(0);   // the trailing out-of-range loads have retired

    // ---- epilogue: fp32 -> output type, store mask of the primer's s5 ----
    // The MFMAs take B as their first operand, so accumulator register
    // 4g + e of lane l holds C[m, n] with m = l % 32 and n = 8g + 4(l / 32) + e
    // inside each 32 x 32 block: four consecutive columns per lane.  Rows past
    // M use an out-of-range offset (dropped by the buffer range check).  Tiles
    // that reach past N, or a C whose rows are not 4-byte aligned, take the
    // element-wise path.
    constexpr int ES = (CT == OUT_F32) ? 4 : 2;
    const char *Cbase = (const char *)p.C + ((int64_t)batch * p.sC + (int64_t)m0 * p.ldc + n0) * ES;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cbase);
    const int ml = lane & 31;
    const int nl = 4 * (lane >> 5);
    const bool vec_store = (n0 + BN <= N) && (((uintptr_t)p.C | (uintptr_t)(p.ldc * ES) | (uintptr_t)(p.sC * ES)) & 3) == 0;
    if (vec_store) {
        // Through LDS, one 32-row block of the wave's sub-tile at a time, so
        // that every global store instruction writes whole row segments:
        // lanes write their four consecutive columns into a row-major block
        // (rows padded by 16 bytes, an odd number of granules, so the 16 rows
        // written at once hit distinct banks), then read it back 16 bytes per
        // lane along the rows and store.
        constexpr int ROWB = WTN * ES + 16;                 // bytes per staged row
        constexpr int CPR = WTN * ES / 16;                  // 16-byte chunks per row
        constexpr int RPI = 64 / CPR;                       // rows per read instruction
        static_assert(RPI * CPR == 64 && 32 % RPI == 0, "row chunks must tile a wave");
        static_assert(NW * 32 * ROWB <= STAGES * STAGE * 16, "epilogue staging fits in LDS");
        __builtin_amdgcn_s_barrier();                       // every wave is done with the stages
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        char *const region = reinterpret_cast<char *>(smem) + wave * 32 * ROWB;
#pragma unroll
        for (int i = 0; i < RM; ++i) {
#pragma unroll
            for (int j = 0; j < RN; ++j) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    char *dst = region + ml * ROWB + (j * 32 + 8 * g + nl) * ES;
                    const float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1];
                    const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
                    if constexpr (CT == OUT_F32) {
                        u32x4 w;
                        w[0] = __builtin_bit_cast(uint32_t, v0);
                        w[1] = __builtin_bit_cast(uint32_t, v1);
                        w[2] = __builtin_bit_cast(uint32_t, v2);
                        w[3] = __builtin_bit_cast(uint32_t, v3);
                        *reinterpret_cast<u32x4 *>(dst) = w;
                    } else {
                        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                        u32x2 w;
                        if constexpr (CT == OUT_F16) {
                            w[0] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v0) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v1) << 16);
                            w[1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v2) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v3) << 16);
                        } else {
                            w[0] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v0) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v1) << 16);
                            w[1] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v2) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v3) << 16);
                        }
                        *reinterpret_cast<u32x2 *>(dst) = w;
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < 32 / RPI; ++t) {
                const int row = t * RPI + lane / CPR, chunk = lane % CPR;
                const u32x4 w = *reinterpret_cast<const u32x4 *>(region + row * ROWB + chunk * 16);
                const int cm = wave_m * WTM + i * 32 + row;
                const int cn = wave_n * WTN + chunk * 16 / ES;
                const uint32_t off = (m0 + cm < M) ? (uint32_t)(cm * p.ldc + cn) * ES : OOB_OFFSET;
                __builtin_amdgcn_raw_buffer_store_b128(w, rc, off, 0, STORE_NT);
                store_data_read(w);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < RM; ++i) {
            const int cm = wave_m * WTM + i * 32 + ml;
            const bool row_ok = m0 + cm < M;
#pragma unroll
            for (int j = 0; j < RN; ++j) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int cn = wave_n * WTN + j * 32 + 8 * (r >> 2) + nl + (r & 3);
                    const uint32_t off = (row_ok && n0 + cn < N) ? (uint32_t)(cm * p.ldc + cn) * ES : OOB_OFFSET;
                    const float v = acc[i][j][r];
                    if constexpr (CT == OUT_F32) {
                        const uint32_t x = __builtin_bit_cast(uint32_t, v);
                        __builtin_amdgcn_raw_buffer_store_b32(x, rc, off, 0, STORE_NT);
                        store_data_read(x);
                    } else if constexpr (CT == OUT_F16) {
                        const uint16_t x = __builtin_bit_cast(uint16_t, (_Float16)v);
                        __builtin_amdgcn_raw_buffer_store_b16(x, rc, off, 0, STORE_NT);
                        store_data_read(x);
                    } else {
                        const uint16_t x = __builtin_bit_cast(uint16_t, (__bf16)v);
                        __builtin_amdgcn_raw_buffer_store_b16(x, rc, off, 0, STORE_NT);
                        store_data_read(x);
                    }
                }
            }
        }
    }
}

}  // namespace tdg
