// gemm_inst.hip -- instantiates the GEMM kernel for one (layout, input type)
// pair; compiled once per pair with -DTDG_TRANSB=0|1 -DTDG_AB=0|1 so the
// instantiations build in parallel.  Exposes one launcher per pair.
#include "gemm_fast.hpp"
#include "gemm_kernel.hpp"
#include "gemm_m16.hpp"
#include "gemm_m16p.hpp"

#ifndef TDG_TRANSB
#error "TDG_TRANSB must be defined"
#endif
#ifndef TDG_AB
#error "TDG_AB must be defined"
#endif

namespace tdg {

template <int KIND, int BM, int BN, int BK, int ST, int WM, int WN, bool TA, bool TB, int CT, bool VEC>
static void launch_one(const GemmArgs &a, int64_t grid, hipStream_t s) {
    if constexpr (KIND == 1) {
        hipLaunchKernelGGL((gemm_fast_kernel<BM, BN, WM, WN, BK, ST, TB, TDG_AB, CT>), dim3((unsigned)grid),
                           dim3(WM * WN * 64), 0, s, a);
    } else if constexpr (KIND == 2) {
        static_assert(BK == 64 || BK == 32, "the 16x16x32 kernel uses K tiles of 64 or 32");
        hipLaunchKernelGGL((gemm_m16_kernel<BM, BN, WM, WN, ST, TA, TB, TDG_AB, CT, false, BK>), dim3((unsigned)grid),
                           dim3(WM * WN * 64), 0, s, a);
    } else if constexpr (KIND == 5) {
        static_assert(BK == 64, "the A window: K tiles of 64");
        hipLaunchKernelGGL((gemm_m16_kernel<BM, BN, WM, WN, ST, TA, TB, TDG_AB, CT, false, 64, true>),
                           dim3((unsigned)grid), dim3(WM * WN * 64), 0, s, a);
    } else if constexpr (KIND == 4) {
        static_assert(BK == 64, "the 16x16x32 kernel uses K tiles of 64");
        hipLaunchKernelGGL((gemm_m16_kernel<BM, BN, WM, WN, ST, TA, TB, TDG_AB, CT, true>), dim3((unsigned)grid),
                           dim3(WM * WN * 64), 0, s, a);
    } else if constexpr (KIND == 3) {
        static_assert(BK == 64, "the 16x16x32 kernel uses K tiles of 64");
        hipLaunchKernelGGL((gemm_m16p_kernel<BM, BN, WM, WN, ST, TA, TB, TDG_AB, CT>), dim3((unsigned)grid),
                           dim3(WM * WN * 64), 0, s, a);
    } else {
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, TB, TDG_AB, CT, VEC>), dim3((unsigned)grid),
                           dim3(NTHREADS), 0, s, a);
    }
}

template <int KIND, int BM, int BN, int BK, int ST, int WM, int WN, bool TA, bool VEC>
static hipError_t launch_ct(int ct, const GemmArgs &a, int64_t grid, hipStream_t s) {
    constexpr bool TB = TDG_TRANSB != 0;
    if constexpr ((KIND >= 1 && !TB && BN / 8 < 16) || (TA && (KIND < 2 || KIND >= 4 || BM / 8 < 16))) {
        // an MC operand needs the direct-to-LDS kernels with >= 128-wide
        // rows; the ping-pong and A-window forms take an A stored M x K only
        return hipErrorInvalidValue;
    } else {
        switch (ct) {
        case OUT_F16: launch_one<KIND, BM, BN, BK, ST, WM, WN, TA, TB, OUT_F16, VEC>(a, grid, s); break;
        case OUT_BF16: launch_one<KIND, BM, BN, BK, ST, WM, WN, TA, TB, OUT_BF16, VEC>(a, grid, s); break;
        default: launch_one<KIND, BM, BN, BK, ST, WM, WN, TA, TB, OUT_F32, VEC>(a, grid, s); break;
        }
        return hipGetLastError();
    }
}

#define TDG_CAT2(a, b) a##b
#define TDG_CAT(a, b) TDG_CAT2(a, b)
#define TDG_LAUNCHER TDG_CAT(TDG_CAT(launch_t, TDG_TRANSB), TDG_CAT(_ab, TDG_AB))

hipError_t TDG_LAUNCHER(int cfg, int ct, int transa, const GemmArgs &a, int64_t grid, hipStream_t s) {
    switch (cfg) {
#define TDG_CASE(ID, KIND, BM, BN, BK, ST, WM, WN, VEC, NAME)                                   \
    case ID:                                                                                     \
        return transa ? launch_ct<KIND, BM, BN, BK, ST, WM, WN, true, VEC>(ct, a, grid, s)     \
                      : launch_ct<KIND, BM, BN, BK, ST, WM, WN, false, VEC>(ct, a, grid, s);
        TDG_CONFIG_LIST(TDG_CASE)
#undef TDG_CASE
    default: return hipErrorInvalidValue;
    }
}

}  // namespace tdg
