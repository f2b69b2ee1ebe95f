// gemm_kernel.hpp -- tiled MFMA GEMM kernel for gfx950 (CDNA4).
//
// One workgroup computes one BM x BN output tile of one problem; the K loop
// runs inside the workgroup with an fp32 accumulator, so no cross-workgroup
// reduction exists (NineToothed GEMM primer, s4: M and N are spread over the
// grid of programs, K stays a loop inside each program).  Per K tile of 64:
//   1. global -> VGPR: each lane fetches 16-byte granules of the A strip
//      (BM x 64) and the B strip; reads past the matrix edges return zero
//      (primer s5 read masks);
//   2. VGPR -> LDS into the buffer not being read (double buffering), in a
//      K-contiguous, XOR-swizzled layout shared by writer and reader (the
//      Croqtile tutorial ch.4 notes that a swizzled store and the operand
//      load must agree on the swizzle);
//   3. LDS -> VGPR operand fragments for v_mfma_f32_32x32x16_{f16,bf16} and
//      the MFMA contraction into AccVGPR-resident accumulators (the
//      fill / load / multiply / store rhythm of Croqtile ch.4, with the
//      accumulator in fp32 as in primer s6);
// then the epilogue converts fp32 to the output type (round to nearest
// even) and stores only elements inside the matrix (primer s5 store mask).
//
// MFMA 32x32x16 operand layout (lane l of 64, 8 sixteen-bit values per lane):
//   A operand: row l % 32, k = 8*(l / 32) + e, e = 0..7
//   B operand: column l % 32, k = 8*(l / 32) + e
//   D (16 fp32 per lane): row 8*(r / 4) + 4*(l / 32) + r % 4, column l % 32.
// Both operands therefore want runs of 8 consecutive k per lane: the LDS
// tiles are stored K-contiguous for A and for B.  For NN (B stored K x N,
// N-contiguous) each lane fetches an 8 x 8 block of B and transposes it in
// registers with byte permutes before writing it to LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.hpp"

namespace tdg {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum { AB_F16 = 0, AB_BF16 = 1 };
enum { OUT_F16 = 0, OUT_BF16 = 1, OUT_F32 = 2 };

constexpr int BK = 64;            // K extent of one staged tile (elements)
constexpr int GRAN = 8;           // elements per 16-byte granule
constexpr int ROW_GRANS = BK / GRAN;
constexpr int NTHREADS = 256;     // four waves per workgroup
constexpr int GROUP_M = 8;        // tile rows per group of the tile order

// LDS position (in granules) of granule g of tile row `row`.  The XOR with
// bits of row and row/8 spreads the 8 rows read by 8 neighbouring lanes, the
// 8 granules of one row written by 8 neighbouring lanes, and the rows 8
// apart written by the NN transpose path over distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int g) {
    return row * ROW_GRANS + (g ^ ((row ^ (row >> 3)) & 7));
}

template <int AB>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (AB == AB_F16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
}

// 8 consecutive elements starting at p, each kept only if its index is in
// [0, lim); lim <= 0 gives zeros.  Used by the predicated (unaligned) path.
__device__ __forceinline__ u32x4 load8_masked(const uint16_t *p, int lim) {
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (i < lim) ? p[i] : (uint16_t)0;
    u32x4 v;
    v[0] = e[0] | ((uint32_t)e[1] << 16);
    v[1] = e[2] | ((uint32_t)e[3] << 16);
    v[2] = e[4] | ((uint32_t)e[5] << 16);
    v[3] = e[6] | ((uint32_t)e[7] << 16);
    return v;
}

// Cache policy of the output stores: non-temporal (the "nt" bit of gfx950's
// buffer stores).  C is written once and never read back by the kernel;
// streaming it past the caches raised the HBM-bound batched TN product with
// fp32 output from 4.38 to 5.36 TB/s (same process, interleaved timing).
constexpr int STORE_NT = 2;

// Called right after a store to global memory with the store's data: keeps
// those registers unchanged until the store has read them (s_waitcnt
// expcnt(0)).  hipcc reuses a store's data registers for the next value as
// soon as the store is issued, and on gfx950 a register write that closely
// follows a store has been seen to reach the store's data (wrong output
// elements, nondeterministically, in an epilogue that stored straight from
// registers); every epilogue store of the library goes through this.
template <class T>
__device__ __forceinline__ void store_data_read(const T &x) {
    asm volatile("s_waitcnt expcnt(0)" ::"v"(x));
}

// The same for a group of stores issued back to back: one wait, after which
// the data registers of every store of the group may be reused (the empty
// statements keep them live until the wait has passed).
template <int N, class T>
__device__ __forceinline__ void store_data_read_all(const T (&x)[N]) {
    asm volatile("s_waitcnt expcnt(0)" ::: "memory");
#pragma unroll
    for (int t = 0; t < N; ++t) asm volatile("" ::"v"(x[t]));
}

template <int CT>
__device__ __forceinline__ void store_out(void *C, int64_t off, float v) {
    if constexpr (CT == OUT_F32) {
        __builtin_nontemporal_store(v, reinterpret_cast<float *>(C) + off);
        store_data_read(v);
    } else if constexpr (CT == OUT_F16) {
        const _Float16 h = (_Float16)v;
        __builtin_nontemporal_store(h, reinterpret_cast<_Float16 *>(C) + off);
        store_data_read(h);
    } else {
        const __bf16 h = (__bf16)v;
        __builtin_nontemporal_store(h, reinterpret_cast<__bf16 *>(C) + off);
        store_data_read(h);
    }
}

// Workgroups are handed to the 8 XCDs round-robin (id % 8); renumbering
// id -> (id % 8) * share + id / 8 makes each XCD walk a contiguous range of
// the `num` logical work items, so tiles that share A rows or B columns meet
// in the same XCD's L2.  A bijection on [0, num) for any num.
__device__ __forceinline__ int xcd_order(int w, int num) {
    const int q = num >> 3, r = num & 7, x = w & 7;
    return x * q + (x < r ? x : r) + (w >> 3);
}

// Logical tile index -> (problem, tile row, tile column).  Tiles are ordered
// in groups of GROUP_M tile rows, column by column inside a group, so a burst
// of concurrent tiles covers a compact block of the output.
template <class Args>
__device__ __forceinline__ void tile_of(const Args &p, int logical, int &batch, int &tm, int &tn) {
    batch = logical / p.tiles_per_batch;
    const int t = logical - batch * p.tiles_per_batch;
    const int group_size = GROUP_M * p.tiles_n;
    const int g = t / group_size;
    const int first_m = g * GROUP_M;
    const int rem = p.tiles_m - first_m;
    const int gm = rem < GROUP_M ? rem : GROUP_M;
    const int in_group = t - g * group_size;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

// Map the workgroup id to (problem, tile row, tile column): one tile per
// workgroup, XCD-aware order over the whole grid.
__device__ __forceinline__ void tile_coords(const GemmArgs &p, int &batch, int &tm, int &tn) {
    tile_of(p, xcd_order(blockIdx.x, gridDim.x), batch, tm, tn);
}

// BM x BN workgroup tile, WM x WN waves, each wave owning a
// (BM/WM) x (BN/WN) sub-tile made of 32 x 32 MFMA tiles.
// TRANSB: false = NN (B is K x N), true = TN (B is N x K).
// VEC: 16-byte vector global loads (requires 16-byte aligned bases, leading
// dimensions and batch strides that are multiples of 8, K % 8 == 0 and, for
// NN, N % 8 == 0); otherwise element loads with per-element masks.
template <int BM, int BN, int WM, int WN, bool TRANSB, int AB, int CT, bool VEC>
__global__ __launch_bounds__(NTHREADS) void gemm_kernel(GemmArgs p) {
    static_assert(WM * WN * 64 == NTHREADS, "four waves per workgroup");
    constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile
    constexpr int RM = WTM / 32, RN = WTN / 32;   // MFMA tiles per wave
    static_assert(RM * 32 == WTM && RN * 32 == WTN, "wave tile must be a multiple of 32");
    constexpr int A_GRANS = BM * ROW_GRANS;       // granules per A stage
    constexpr int B_GRANS = BN * ROW_GRANS;
    constexpr int GA = A_GRANS / NTHREADS;        // A granules per lane
    static_assert(GA * NTHREADS == A_GRANS, "A tile must split evenly");
    // TN: B granules per lane, like A.  NN: 8 x 8 blocks, BN of them.
    constexpr int GB_TN = B_GRANS / NTHREADS;
    constexpr int NB_NN = (BN + NTHREADS - 1) / NTHREADS;   // NN blocks per lane
    constexpr int STAGE = A_GRANS + B_GRANS;

    __shared__ u32x4 smem[2 * STAGE];

    int batch, tm, tn;
    tile_coords(p, batch, tm, tn);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_m = wave / WN, wave_n = wave % WN;

    const int M = p.M, N = p.N, K = p.K;
    const int m0 = tm * BM, n0 = tn * BN;
    const uint16_t *Ab = p.A + (int64_t)batch * p.sA;
    const uint16_t *Bb = p.B + (int64_t)batch * p.sB;

    // ---- per-lane global fetch descriptors (fixed over the K loop) ----
    const uint16_t *a_ptr[GA];
    bool a_row_ok[GA];
    int a_lds[GA];
    int a_kof[GA];
#pragma unroll
    for (int q = 0; q < GA; ++q) {
        const int idx = tid + q * NTHREADS;
        const int row = idx / ROW_GRANS, g = idx % ROW_GRANS;
        const int grow = m0 + row;
        a_row_ok[q] = grow < M;
        a_ptr[q] = Ab + (int64_t)(a_row_ok[q] ? grow : 0) * p.lda + g * GRAN;
        a_kof[q] = g * GRAN;
        a_lds[q] = swz(row, g);
    }

    constexpr int GBL = TRANSB ? GB_TN : NB_NN * 8;   // B vectors per lane
    const uint16_t *b_ptr[TRANSB ? GB_TN : NB_NN];
    bool b_ok[TRANSB ? GB_TN : NB_NN];
    int b_lds[TRANSB ? GB_TN : NB_NN];
    int b_kof[TRANSB ? GB_TN : NB_NN];
    int b_ncnt[TRANSB ? GB_TN : NB_NN];
    if constexpr (TRANSB) {
#pragma unroll
        for (int q = 0; q < GB_TN; ++q) {
            const int idx = tid + q * NTHREADS;
            const int row = idx / ROW_GRANS, g = idx % ROW_GRANS;
            const int gn = n0 + row;
            b_ok[q] = gn < N;
            b_ptr[q] = Bb + (int64_t)(b_ok[q] ? gn : 0) * p.ldb + g * GRAN;
            b_kof[q] = g * GRAN;
            b_lds[q] = swz(row, g);
            b_ncnt[q] = 0;
        }
    } else {
        // block b -> (kb, nb): k rows kb*8..kb*8+7, columns nb*8..nb*8+7
#pragma unroll
        for (int q = 0; q < NB_NN; ++q) {
            const int b = tid + q * NTHREADS;
            const int kb = b / (BN / 8), nb = b % (BN / 8);
            const int gn = n0 + nb * 8;
            b_ok[q] = (b < BN) && (gn < N);
            b_ncnt[q] = N - gn;                        // valid columns in this block
            b_ptr[q] = Bb + (int64_t)(kb * 8) * p.ldb + (b_ok[q] ? gn : 0);
            b_kof[q] = kb * 8;
            b_lds[q] = 0;                              // NN blocks are placed in stash()
        }
    }

    u32x4 ra[GA];
    u32x4 rb[GBL];

    auto fetch = [&](int k0) {
#pragma unroll
        for (int q = 0; q < GA; ++q) {
            const int kk = k0 + a_kof[q];
            if constexpr (VEC) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (a_row_ok[q] && kk < K) v = *reinterpret_cast<const u32x4 *>(a_ptr[q] + k0);
                ra[q] = v;
            } else {
                ra[q] = load8_masked(a_ptr[q] + k0, a_row_ok[q] ? K - kk : 0);
            }
        }
        if constexpr (TRANSB) {
#pragma unroll
            for (int q = 0; q < GB_TN; ++q) {
                const int kk = k0 + b_kof[q];
                if constexpr (VEC) {
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (b_ok[q] && kk < K) v = *reinterpret_cast<const u32x4 *>(b_ptr[q] + k0);
                    rb[q] = v;
                } else {
                    rb[q] = load8_masked(b_ptr[q] + k0, b_ok[q] ? K - kk : 0);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < NB_NN; ++q) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int kk = k0 + b_kof[q] + i;
                    const uint16_t *src = b_ptr[q] + (int64_t)(k0 + i) * p.ldb;
                    if constexpr (VEC) {
                        u32x4 v = {0u, 0u, 0u, 0u};
                        if (b_ok[q] && kk < K) v = *reinterpret_cast<const u32x4 *>(src);
                        rb[q * 8 + i] = v;
                    } else {
                        rb[q * 8 + i] = load8_masked(src, (b_ok[q] && kk < K) ? b_ncnt[q] : 0);
                    }
                }
            }
        }
    };

    auto stash = [&](int stage) {
        u32x4 *sa = smem + stage * STAGE;
        u32x4 *sb = sa + A_GRANS;
#pragma unroll
        for (int q = 0; q < GA; ++q) sa[a_lds[q]] = ra[q];
        if constexpr (TRANSB) {
#pragma unroll
            for (int q = 0; q < GB_TN; ++q) sb[b_lds[q]] = rb[q];
        } else {
#pragma unroll
            for (int q = 0; q < NB_NN; ++q) {
                const int b = tid + q * NTHREADS;
                if (b < BN) {
                    const int kb = b / (BN / 8), nb = b % (BN / 8);
                    // transpose the 8 (k) x 8 (n) block: output c holds column
                    // nb*8+c as 8 consecutive k values (2 per dword).
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const unsigned sel = (c & 1) ? 0x07060302u : 0x05040100u;
                        u32x4 o;
#pragma unroll
                        for (int d = 0; d < 4; ++d)
                            o[d] = __builtin_amdgcn_perm(rb[q * 8 + 2 * d + 1][c >> 1],
                                                         rb[q * 8 + 2 * d][c >> 1], sel);
                        sb[swz(nb * 8 + c, kb)] = o;
                    }
                }
            }
        }
    };

    f32x16 acc[RM][RN];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (K + BK - 1) / BK;
    const int frag_row = lane & 31;
    const int frag_g = lane >> 5;
    if (nk > 0) {
        fetch(0);
        stash(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool has_next = kt + 1 < nk;
            if (has_next) fetch((kt + 1) * BK);
            const u32x4 *sa = smem + cur * STAGE;
            const u32x4 *sb = sa + A_GRANS;
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                u32x4 af[RM], bf[RN];
                const int g = kk * 2 + frag_g;
#pragma unroll
                for (int i = 0; i < RM; ++i) af[i] = sa[swz(wave_m * WTM + i * 32 + frag_row, g)];
#pragma unroll
                for (int j = 0; j < RN; ++j) bf[j] = sb[swz(wave_n * WTN + j * 32 + frag_row, g)];
#pragma unroll
                for (int i = 0; i < RM; ++i)
#pragma unroll
                    for (int j = 0; j < RN; ++j) acc[i][j] = mfma_32x32x16<AB>(af[i], bf[j], acc[i][j]);
            }
            if (has_next) stash(cur ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue: fp32 -> output type, masked store ----
    void *Cb = (char *)p.C + (int64_t)batch * p.sC * (CT == OUT_F32 ? 4 : 2);
    const int col_l = lane & 31;
    const int row_l = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
        for (int j = 0; j < RN; ++j) {
            const int gn = n0 + wave_n * WTN + j * 32 + col_l;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wave_m * WTM + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                if (gm < M && gn < N) store_out<CT>(Cb, (int64_t)gm * p.ldc + gn, acc[i][j][r]);
            }
        }
    }
}

}  // namespace tdg
