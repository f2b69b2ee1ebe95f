// gemm_fast.hpp -- the vectorised MFMA GEMM kernel for gfx950 (aligned operands).
//
// Same decomposition as the general kernel (one workgroup per output tile,
// K loop inside the workgroup, fp32 accumulators; NineToothed GEMM primer s4),
// built on three gfx950 features:
//
//  * Direct global -> LDS loads in buffer form (buffer_load_dwordx4 ... lds).
//    Lane l of an instruction writes its 16 bytes at LDS base + 16*l, so the
//    swizzled LDS layout is produced by choosing, for each LDS slot, which
//    global granule its lane fetches.  A lane whose element lies outside the
//    matrix uses an offset past the buffer's range: the hardware skips the
//    memory access and writes zeros, which is exactly the zero-filled masked
//    read of the primer's s5, with no branch and no staging registers.
//  * v_mfma_f32_32x32x16_{f16,bf16} with AccVGPR accumulators.
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
// distinct 16-byte bank groups (the LDS has 64 four-byte banks), so the
// operand reads are conflict-free; the direct loads write 1 KiB contiguous
// runs.  Writer and reader derive positions from the same formulas (the
// Croqtile tutorial ch.4 notes that a swizzled store and the operand load
// must agree on the swizzle).
//
// Pipeline: the STAGES LDS stages are separate objects, so the compiler can
// prove that reading one stage never touches the direct loads in flight into
// the others.  Loads run STAGES-1 tiles ahead; the fragments of K step kk+1
// are read while the MFMAs of step kk run; the single barrier per K tile sits
// before the tile's last step, whose fragments are already in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.hpp"
#include "gemm_kernel.hpp"

namespace tdg {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

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
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"(lds_addr)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
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

// s_waitcnt immediate (gfx9 encoding): wait until at most VM vector memory
// operations are outstanding and every LDS operation has completed.
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
}

// Order the instructions of one compute block: MF MFMAs with DS LDS reads
// and VM direct global loads spread between them (LDS reads first), PER
// MFMAs before each memory instruction (a scheduling constraint only; it
// changes no result).
template <int MF, int DS, int VM, int PER>
__device__ __forceinline__ void interleave_rec() {
    if constexpr (MF > 0 || DS > 0 || VM > 0) {
        constexpr int take = MF < PER ? MF : PER;
        if constexpr (take > 0) __builtin_amdgcn_sched_group_barrier(0x008, take, 0);
        if constexpr (DS > 0) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            interleave_rec<MF - take, DS - 1, VM, PER>();
        } else if constexpr (VM > 0) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            interleave_rec<MF - take, 0, VM - 1, PER>();
        } else {
            interleave_rec<MF - take, 0, 0, PER>();
        }
    }
}

template <int NMF, int NDS, int NVM>
__device__ __forceinline__ void interleave_hint() {
    constexpr int MEM = NDS + NVM;
    constexpr int PER = MEM > 0 ? (NMF > MEM ? NMF / MEM : 1) : NMF;
    interleave_rec<NMF, NDS, NVM, PER>();
}

// Compile-time loop: f(std::integral_constant<int, i>) for i in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <int BM, int BN, int WM, int WN, int BK, int STAGES, bool TRANSB, int AB, int CT>
__global__ __launch_bounds__(WM * WN * 64) void gemm_fast_kernel(GemmArgs p) {
    constexpr int NT = WM * WN * 64, NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int RM = WTM / 32, RN = WTN / 32;
    static_assert(RM * 32 == WTM && RN * 32 == WTN, "wave tile must be a multiple of 32");
    static_assert(BK == 32 || BK == 64, "BK is 32 or 64");
    static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 stages");
    constexpr int KG = BK / GRAN;                    // granules per K-contiguous row
    constexpr int KS = BK / 16;                      // MFMA K steps per tile
    constexpr int A_SLOTS = BM * KG;                 // granules of one A stage
    constexpr int B_SLOTS = BN * KG;                 // granules of one B stage (BK x BN either way)
    constexpr int STAGE = A_SLOTS + B_SLOTS;
    constexpr int A_INST = A_SLOTS / NT;             // direct loads per lane per stage
    constexpr int B_INST = B_SLOTS / NT;
    static_assert(A_INST * NT == A_SLOTS && B_INST * NT == B_SLOTS, "tile must split over the lanes");
    constexpr int NDMA = A_INST + B_INST;
    constexpr int BNG = BN / GRAN;                   // granules per NN B row
    static_assert(TRANSB || BNG >= 16, "NN B swizzle needs rows of at least 16 granules");
    static_assert((STAGES - 1) * NDMA < 64, "vmcnt range");

    __shared__ u32x4 sm0[STAGE];
    __shared__ u32x4 sm1[STAGE];
    __shared__ u32x4 sm2[STAGES > 2 ? STAGE : 1];
    __shared__ u32x4 sm3[STAGES > 3 ? STAGE : 1];
    auto stage_ptr = [&](auto tag) -> u32x4 * {
        constexpr int s = decltype(tag)::value;
        if constexpr (s == 0) return sm0;
        else if constexpr (s == 1) return sm1;
        else if constexpr (s == 2) return sm2;
        else return sm3;
    };

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
    uint32_t a_off[A_INST];
    int a_klim[A_INST];      // loaded while k0 < a_klim (K - 8g; -1 if the row is outside)
#pragma unroll
    for (int q = 0; q < A_INST; ++q) {
        const int slot = (q * NW + wave) * 64 + lane;
        const int row = slot / KG, phys = slot % KG;
        const int g = kpos<BK>(row, phys) - row * KG;   // the XOR is an involution
        a_off[q] = (uint32_t)(row * p.lda + g * GRAN) * 2u;
        a_klim[q] = (m0 + row < M) ? K - g * GRAN : -1;
    }
    uint32_t b_off[B_INST];
    int b_klim[B_INST];
#pragma unroll
    for (int q = 0; q < B_INST; ++q) {
        const int slot = (q * NW + wave) * 64 + lane;
        if constexpr (TRANSB) {
            const int row = slot / KG, phys = slot % KG;
            const int g = kpos<BK>(row, phys) - row * KG;
            b_off[q] = (uint32_t)(row * p.ldb + g * GRAN) * 2u;
            b_klim[q] = (n0 + row < N) ? K - g * GRAN : -1;
        } else {
            const int k = slot / BNG, phys = slot % BNG;
            const int c = npos<BNG>(k, phys) - k * BNG;
            b_off[q] = (uint32_t)(k * p.ldb + c * GRAN) * 2u;
            b_klim[q] = (n0 + c * GRAN < N) ? K - k : -1;
        }
    }

    // Enqueue the direct loads of K tile kt into the stage at sa.
    auto issue_to = [&](int kt, u32x4 *sa) {
        const int k0 = kt * BK;
        const u32x4 ra = rsrc_words(Atile + k0);
        const u32x4 rb = rsrc_words(TRANSB ? Btile + k0 : Btile + (int64_t)k0 * p.ldb);
        const uint32_t la = lds_addr_of(sa) + (uint32_t)wave * 1024u;
        const uint32_t lb = la + A_SLOTS * 16u;
#pragma unroll
        for (int q = 0; q < A_INST; ++q) {
            const uint32_t off = (k0 < a_klim[q]) ? a_off[q] : OOB_OFFSET;
            dma16(ra, off, la + q * NW * 1024u);
        }
#pragma unroll
        for (int q = 0; q < B_INST; ++q) {
            const uint32_t off = (k0 < b_klim[q]) ? b_off[q] : OOB_OFFSET;
            dma16(rb, off, lb + q * NW * 1024u);
        }
    };

    // Direct load number q (0 <= q < NDMA) of K tile kt into the stage at sa.
    auto dma_op = [&](auto qtag, int kt, u32x4 *sa) {
        constexpr int q = decltype(qtag)::value;
        const int k0 = kt * BK;
        const uint32_t la = lds_addr_of(sa) + (uint32_t)wave * 1024u;
        if constexpr (q < A_INST) {
            const uint32_t off = (k0 < a_klim[q]) ? a_off[q] : OOB_OFFSET;
            dma16(rsrc_words(Atile + k0), off, la + q * NW * 1024u);
        } else {
            constexpr int qb = q - A_INST;
            const uint32_t off = (k0 < b_klim[qb]) ? b_off[qb] : OOB_OFFSET;
            dma16(rsrc_words(TRANSB ? Btile + k0 : Btile + (int64_t)k0 * p.ldb), off,
                  la + A_SLOTS * 16u + qb * NW * 1024u);
        }
    };

    // ---- fragment addresses within a stage (granules for b128 reads, bytes
    // for the NN B transposing reads) ----
    const int frag_row = lane & 31;
    const int frag_g = lane >> 5;
    int a_frag[RM][KS];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) a_frag[i][kk] = kpos<BK>(wave_m * WTM + i * 32 + frag_row, kk * 2 + frag_g);
    int b_frag[RN][KS][TRANSB ? 1 : 2];
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            if constexpr (TRANSB) {
                b_frag[j][kk][0] = kpos<BK>(wave_n * WTN + j * 32 + frag_row, kk * 2 + frag_g);
            } else {
                const int grp = lane >> 4, pos = lane & 15;
                const int jr = pos >> 2, q4 = pos & 3;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = kk * 16 + 8 * (grp >> 1) + 4 * h + jr;
                    const int n = wave_n * WTN + j * 32 + 16 * (grp & 1) + 4 * q4;
                    const int c = n / GRAN, half = (n % GRAN) / 4;
                    b_frag[j][kk][h] = npos<BNG>(k, c) * 16 + half * 8;
                }
            }
        }

    // MFMA operand fragments of K step kk from the stage at sa.
    auto frags_from = [&](const u32x4 *sa, int kk, u32x4 (&af)[RM], u32x4 (&bf)[RN]) {
        const u32x4 *sb = sa + A_SLOTS;
#pragma unroll
        for (int i = 0; i < RM; ++i) af[i] = sa[a_frag[i][kk]];
#pragma unroll
        for (int j = 0; j < RN; ++j) {
            if constexpr (TRANSB) {
                bf[j] = sb[b_frag[j][kk][0]];
            } else {
                const char *base = reinterpret_cast<const char *>(sb);
                s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(base + b_frag[j][kk][0]));
                s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(base + b_frag[j][kk][1]));
                u32x4 v;
                v[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
                v[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
                v[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
                v[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
                bf[j] = v;
            }
        }
    };

    // LDS read number d (0 <= d < RM + RN or RM + 2 RN) of K step kk's fragments.
    auto frag_op = [&](auto dtag, const u32x4 *sa, int kk, u32x4 (&af)[RM], u32x4 (&bf)[RN]) {
        constexpr int d = decltype(dtag)::value;
        const u32x4 *sb = sa + A_SLOTS;
        if constexpr (d < RM) {
            af[d] = sa[a_frag[d][kk]];
        } else if constexpr (TRANSB) {
            bf[d - RM] = sb[b_frag[d - RM][kk][0]];
        } else {
            constexpr int j = (d - RM) / 2, h = (d - RM) % 2;
            const char *base = reinterpret_cast<const char *>(sb);
            const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(base + b_frag[j][kk][h]));
            const uint64_t w = __builtin_bit_cast(uint64_t, v);
            bf[j][2 * h] = (uint32_t)w;
            bf[j][2 * h + 1] = (uint32_t)(w >> 32);
        }
    };

    f32x16 acc[RM][RN];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    constexpr int NDS = RM + (TRANSB ? RN : 2 * RN);   // LDS reads per K step
    constexpr int NMF = RM * RN;                       // MFMAs per K step
    const int nk = (K + BK - 1) / BK;
    u32x4 af[2][RM], bf[2][RN];

    // Loads of tiles past the last one are all out of range: they fetch
    // nothing and only write zeros into a stage that is never read again.
    if (nk > 0) {
        issue_to(0, sm0);
        issue_to(1, sm1);
        if constexpr (STAGES > 2) issue_to(2, sm2);
        if constexpr (STAGES > 3) issue_to(3, sm3);
        wait_vm_lgkm0<(STAGES - 1) * NDMA>();    // tile 0 has landed (this lane)
        __builtin_amdgcn_s_barrier();             // ... for every lane
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        frags_from(sm0, 0, af[0], bf[0]);
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
                    acc[i][j] = mfma_32x32x16<AB>(af[kk & 1][i], bf[kk & 1][j], acc[i][j]);
            interleave_hint<NMF, NDS, 0>();
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
                acc[i][j] = mfma_32x32x16<AB>(af[(KS - 1) & 1][i], bf[(KS - 1) & 1][j], acc[i][j]);
            });
            static_for<s0 * NDS / NSUB, (s0 + 1) * NDS / NSUB>([&](auto d) {
                frag_op(d, nxt, 0, af[KS & 1], bf[KS & 1]);
            });
            dma_op(sub, kt + STAGES, cur);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    for (int kt = 0; kt < nk; kt += STAGES) {
        tile_iter(std::integral_constant<int, 0>{}, kt);
        if (kt + 1 < nk) tile_iter(std::integral_constant<int, 1>{}, kt + 1);
        if constexpr (STAGES > 2) {
            if (kt + 2 < nk) tile_iter(std::integral_constant<int, 2>{}, kt + 2);
        }
        if constexpr (STAGES > 3) {
            if (kt + 3 < nk) tile_iter(std::integral_constant<int, 3>{}, kt + 3);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);   // the trailing out-of-range loads have retired

    // ---- epilogue: fp32 -> output type; out-of-range elements are dropped by
    // the buffer range check (store mask of the primer's s5) ----
    constexpr int ES = (CT == OUT_F32) ? 4 : 2;
    const char *Cbase = (const char *)p.C + ((int64_t)batch * p.sC + (int64_t)m0 * p.ldc + n0) * ES;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cbase);
    const int col_l = lane & 31;
    const int row_l = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
        for (int j = 0; j < RN; ++j) {
            // one 32 x 32 tile at a time: keeps the conversion temporaries few
            __builtin_amdgcn_sched_barrier(0);
            const int cn = wave_n * WTN + j * 32 + col_l;
            const bool col_ok = n0 + cn < N;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int cm = wave_m * WTM + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                const uint32_t off = (col_ok && m0 + cm < M) ? (uint32_t)(cm * p.ldc + cn) * ES : OOB_OFFSET;
                const float v = acc[i][j][r];
                if constexpr (CT == OUT_F32) {
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rc, off, 0, 0);
                } else if constexpr (CT == OUT_F16) {
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)v), rc, off, 0, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)v), rc, off, 0, 0);
                }
            }
        }
    }
}

}  // namespace tdg
