// gemm_f8_inst.hip -- instantiates the 8-bit GEMM kernel for one pair of
// operand formats; compiled once per pair with -DTDG_FA=0|1 -DTDG_FB=0|1
// (0 = E4M3, 1 = E5M2) so the instantiations build in parallel.  Exposes
// one launcher per pair.
#include "gemm_f8.hpp"

#ifndef TDG_FA
#error "TDG_FA must be defined"
#endif
#ifndef TDG_FB
#error "TDG_FB must be defined"
#endif

namespace tdg {

template <int BM, int BN, int ST, int WM, int WN, bool BS, int CT>
static void launch_f8_one(const F8Args &a, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_f8_kernel<BM, BN, WM, WN, ST, TDG_FA, TDG_FB, BS, CT>), dim3((unsigned)grid),
                       dim3(WM * WN * 64), 0, s, a);
}

template <int BM, int BN, int ST, int WM, int WN, bool BS>
static hipError_t launch_f8_ct(int ct, const F8Args &a, int64_t grid, hipStream_t s) {
    switch (ct) {
    case OUT_F16: launch_f8_one<BM, BN, ST, WM, WN, BS, OUT_F16>(a, grid, s); break;
    case OUT_BF16: launch_f8_one<BM, BN, ST, WM, WN, BS, OUT_BF16>(a, grid, s); break;
    default: launch_f8_one<BM, BN, ST, WM, WN, BS, OUT_F32>(a, grid, s); break;
    }
    return hipGetLastError();
}

#define TDG_CAT2(a, b) a##b
#define TDG_CAT(a, b) TDG_CAT2(a, b)
#define TDG_F8_LAUNCHER TDG_CAT(TDG_CAT(launch_f8_a, TDG_FA), TDG_CAT(_b, TDG_FB))

// bscale: whether block scales are given (for A, B or both).
hipError_t TDG_F8_LAUNCHER(int cfg, int ct, int bscale, const F8Args &a, int64_t grid, hipStream_t s) {
    switch (cfg) {
#define TDG_F8_CASE(ID, BM, BN, ST, WM, WN, NAME)                                       \
    case ID:                                                                             \
        return bscale ? launch_f8_ct<BM, BN, ST, WM, WN, true>(ct, a, grid, s)          \
                      : launch_f8_ct<BM, BN, ST, WM, WN, false>(ct, a, grid, s);
        TDG_F8_CONFIG_LIST(TDG_F8_CASE)
#undef TDG_F8_CASE
    default: return hipErrorInvalidValue;
    }
}

}  // namespace tdg
