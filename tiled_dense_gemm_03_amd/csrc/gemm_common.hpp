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
};

}  // namespace tdg

// X(id, BM, BN, WM, WN, VEC, name): BM x BN workgroup tile (BK = 64),
// WM x WN waves, VEC = vectorised loads (aligned operands) or the
// predicated element-load path.
#define TDG_CONFIG_LIST(X)                                   \
    X(0, 256, 256, 2, 2, true, "256x256x64_w2x2_vec")        \
    X(1, 256, 128, 2, 2, true, "256x128x64_w2x2_vec")        \
    X(2, 128, 256, 2, 2, true, "128x256x64_w2x2_vec")        \
    X(3, 128, 128, 2, 2, true, "128x128x64_w2x2_vec")        \
    X(4, 64, 64, 2, 2, true, "64x64x64_w2x2_vec")            \
    X(5, 64, 64, 2, 2, false, "64x64x64_w2x2_pred")          \
    X(6, 128, 128, 2, 2, false, "128x128x64_w2x2_pred")
