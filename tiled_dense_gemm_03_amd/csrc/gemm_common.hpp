// gemm_common.hpp -- definitions shared by the host API and the kernels:
// the kernel argument block and the table of compiled tile configurations.
#pragma once
#include <stdint.h>

namespace tdg {

// Kernel arguments (passed by value).  Strides are in elements.
struct GemmArgs {
    const uint16_t *A;
    const uint16_t *B;
    void *C;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;          // batch strides; 0 for a single problem
    int M, N, K;
    int tiles_m, tiles_n;
    int tiles_per_batch;
    // Split-K schedule of the 16x16x32 kernel (ignored by the others):
    // workgroups [0, dp_tiles) each own one whole tile; the remaining
    // workgroups are sk_split K slices of each of the last tiles.  ws holds
    // one fp32 partial tile per slice, ws_flags one arrival counter per
    // split tile (zero between calls).
    float *ws;
    int *ws_flags;
    int dp_tiles;
    int sk_split;
};

// Kernel arguments of the 8-bit product C = A * B^T (A M x K, B N x K, both
// K-contiguous; strides in elements = bytes for A and B).
struct F8Args {
    const uint8_t *A;
    const uint8_t *B;
    void *C;
    int64_t lda, ldb, ldc;
    const uint8_t *xa, *xb;      // E8M0 scales, one byte per row and 32-element K block (or null)
    int64_t ldxa, ldxb;          // bytes between rows of xa / xb (multiples of 4)
    const float *sa, *sb;        // fp32 scales per row of A / row of B (or null)
    int64_t inc_sa, inc_sb;      // 0: one scale for every row
    int M, N, K;
    int tiles_m, tiles_n;
    int tiles_per_batch;         // tiles_m * tiles_n (one problem)
};

}  // namespace tdg

// X(id, KIND, BM, BN, BK, ST, WM, WN, VEC, name): ids run 0, 1, 2, ... in
// list order (checked at compile time).  BM x BN workgroup tile, WM x WN
// waves.  KIND 1 = the direct-to-LDS kernel (aligned operands only) with K
// tiles of BK and ST pipeline stages; KIND 0 = the register-staged kernel
// (BK 64, two stages), VEC = vectorised loads (aligned operands) or the
// predicated element-load path (any operands); KIND 2 = the direct-to-LDS
// kernel built on 16 x 16 x 32 MFMAs (aligned operands, BK 64 or 32); KIND 3 = its
// persistent form (one workgroup per CU walking its tiles, K > 0); KIND 4 =
// its ping-pong form (two groups of four waves alternating a memory phase
// and an MFMA phase; A stored M x K only); KIND 5 = the 16 x 16 x 32 kernel
// with A's rows loaded as aligned 128-byte chunks into a ring of three slots
// (for an A whose rows do not start on 128-byte lines; A stored M x K only).
#define TDG_CONFIG_LIST(X)                                                   \
    X(0, 1, 256, 256, 64, 2, 2, 4, true, "256x256x64_s2_w2x4_lds")           \
    X(1, 1, 256, 256, 32, 3, 2, 4, true, "256x256x32_s3_w2x4_lds")           \
    X(2, 1, 256, 256, 32, 3, 2, 2, true, "256x256x32_s3_w2x2_lds")           \
    X(3, 1, 256, 128, 64, 2, 2, 2, true, "256x128x64_s2_w2x2_lds")           \
    X(4, 1, 128, 128, 64, 2, 2, 2, true, "128x128x64_s2_w2x2_lds")           \
    X(5, 1, 128, 128, 32, 4, 2, 2, true, "128x128x32_s4_w2x2_lds")           \
    X(6, 0, 128, 128, 64, 2, 2, 2, true, "128x128x64_w2x2_vec")              \
    X(7, 0, 64, 64, 64, 2, 2, 2, true, "64x64x64_w2x2_vec")                  \
    X(8, 0, 64, 64, 64, 2, 2, 2, false, "64x64x64_w2x2_pred")                \
    X(9, 0, 128, 128, 64, 2, 2, 2, false, "128x128x64_w2x2_pred")           \
    X(10, 2, 256, 256, 64, 2, 2, 4, true, "256x256x64_s2_w2x4_m16")          \
    X(11, 2, 128, 128, 64, 4, 2, 2, true, "128x128x64_s4_w2x2_m16")          \
    X(12, 2, 128, 128, 64, 4, 2, 4, true, "128x128x64_s4_w2x4_m16")          \
    X(13, 2, 128, 128, 64, 2, 2, 2, true, "128x128x64_s2_w2x2_m16")          \
    X(14, 3, 256, 256, 64, 2, 2, 4, true, "256x256x64_s2_w2x4_m16p")         \
    X(15, 2, 256, 256, 64, 2, 2, 2, true, "256x256x64_s2_w2x2_m16")          \
    X(16, 4, 256, 256, 64, 2, 2, 4, true, "256x256x64_s2_w2x4_m16pp")        \
    X(17, 2, 256, 256, 32, 4, 2, 4, true, "256x256x32_s4_w2x4_m16")          \
    X(18, 5, 256, 256, 64, 2, 2, 4, true, "256x256x64_s2_w2x4_m16aw")        \
    X(19, 5, 128, 128, 64, 4, 2, 4, true, "128x128x64_s4_w2x4_m16aw")

// 8-bit configurations: X(id, BM, BN, STAGES, WM, WN, name), K tiles of 128.
#define TDG_F8_CONFIG_LIST(X)                                   \
    X(0, 256, 256, 2, 2, 4, "f8_256x256x128_s2_w2x4")          \
    X(1, 128, 128, 4, 2, 2, "f8_128x128x128_s4_w2x2")
