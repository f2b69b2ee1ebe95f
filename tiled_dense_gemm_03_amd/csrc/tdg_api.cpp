// tdg_api.cpp -- the C ABI of the tiled dense GEMM library (host side).
//
// Validates arguments, picks a tile configuration and enqueues exactly one
// kernel on the caller's stream.  No allocation, no synchronisation, no
// per-call state beyond the thread-local error text and a per-device
// architecture check made once.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/tdg.h"
#include "gemm_common.hpp"

namespace tdg {

hipError_t launch_t0_ab0(int cfg, int ct, const GemmArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_t0_ab1(int cfg, int ct, const GemmArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_t1_ab0(int cfg, int ct, const GemmArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_t1_ab1(int cfg, int ct, const GemmArgs &a, int64_t grid, hipStream_t s);

namespace {

struct Config {
    int kind, bm, bn, bk, stages, wm, wn;
    bool vec;
    const char *name;
};

const Config kConfigs[] = {
#define TDG_ROW(ID, KIND, BM, BN, BK, ST, WM, WN, VEC, NAME) {KIND, BM, BN, BK, ST, WM, WN, VEC, NAME},
    TDG_CONFIG_LIST(TDG_ROW)
#undef TDG_ROW
};
constexpr int kNumConfigs = (int)(sizeof(kConfigs) / sizeof(kConfigs[0]));

constexpr int kConfigIds[] = {
#define TDG_ID(ID, KIND, BM, BN, BK, ST, WM, WN, VEC, NAME) ID,
    TDG_CONFIG_LIST(TDG_ID)
#undef TDG_ID
};
constexpr bool ids_in_order(int i) { return i == kNumConfigs || (kConfigIds[i] == i && ids_in_order(i + 1)); }
static_assert(ids_in_order(0), "configuration ids must be 0, 1, 2, ... in list order");

thread_local char g_err[512] = "";

tdg_status fail(tdg_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

// Architecture check, once per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

tdg_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(TDG_NOT_SUPPORTED, "no HIP device is current");
    if (dev < 0 || dev >= kMaxDevices) return fail(TDG_NOT_SUPPORTED, "device index %d out of range", dev);
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(TDG_NOT_SUPPORTED, "cannot query device %d", dev);
        st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_release);
        if (st != 1) return fail(TDG_NOT_SUPPORTED, "device %d is %s, this library targets gfx950", dev,
                                 prop.gcnArchName);
    }
    if (st != 1) return fail(TDG_NOT_SUPPORTED, "device %d is not gfx950", dev);
    return TDG_SUCCESS;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Whether the vectorised path may serve these operands: 16-byte aligned
// bases, row strides and batch strides that keep every 8-element granule
// aligned, and contiguous extents (K for A and TN-B, N for NN-B) that are
// whole granules.
bool vec_ok(int transb, int64_t N, int64_t K, const void *A, int64_t lda, int64_t sA,
            const void *B, int64_t ldb, int64_t sB, int64_t batch) {
    if (!aligned16(A) || !aligned16(B)) return false;
    if ((lda & 7) || (ldb & 7) || (K & 7)) return false;
    if (!transb && (N & 7)) return false;
    if (batch > 1 && ((sA & 7) || (sB & 7))) return false;
    return true;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Whether configuration `cf` can serve the operands: the vectorised kinds
// need vec_ok; the direct-to-LDS kinds also need every in-tile byte offset
// below 2^31 (buffer offsets are 32-bit) and, for NN, B rows of at least 16
// granules in LDS.
bool config_ok(const Config &cf, int transb, bool vec, int64_t lda, int64_t ldb, int64_t ldc, int c_type) {
    if (!cf.vec) return true;
    if (!vec) return false;
    if (cf.kind < 1) return true;
    const int64_t lim = (int64_t)1 << 31;
    const int64_t es = (c_type == TDG_F32) ? 4 : 2;
    if ((int64_t)cf.bm * lda * 2 >= lim || (int64_t)cf.bm * ldc * es >= lim) return false;
    if (transb ? (int64_t)cf.bn * ldb * 2 >= lim : (int64_t)cf.bk * ldb * 2 >= lim) return false;
    if (!transb && cf.bn / 8 < 16) return false;
    return true;
}

int config_by_name(const char *name) {
    for (int i = 0; i < kNumConfigs; ++i)
        if (strcmp(kConfigs[i].name, name) == 0) return i;
    return -1;
}

// Tile-configuration choice (measured on MI355X): 256 x 256 tiles on the
// 16 x 16 x 32 MFMA kernel when the problem has at least one tile per CU
// (256); 128 x 128 tiles for smaller problems; the register-staged kernel
// when the direct-load kernels cannot address the operands; the predicated
// kernel for misaligned operands.
int choose(int transb, bool vec, int64_t M, int64_t N, int64_t batch, int64_t lda, int64_t ldb, int64_t ldc,
           int c_type) {
    const int64_t b = batch < 1 ? 1 : batch;
    if (vec) {
        const int64_t tiles256 = cdiv(M, 256) * cdiv(N, 256) * b;
        const int id = config_by_name("256x256x64_s2_w2x4_m16");
        if (tiles256 >= 256 && config_ok(kConfigs[id], transb, vec, lda, ldb, ldc, c_type)) return id;
        const int small = config_by_name("128x128x64_s2_w2x2_lds");
        if (config_ok(kConfigs[small], transb, vec, lda, ldb, ldc, c_type)) return small;
        return config_by_name((cdiv(M, 128) * cdiv(N, 128) * b >= 256) ? "128x128x64_w2x2_vec" : "64x64x64_w2x2_vec");
    }
    return config_by_name((cdiv(M, 128) * cdiv(N, 128) * b >= 256) ? "128x128x64_w2x2_pred" : "64x64x64_w2x2_pred");
}

tdg_status validate(int transb, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t sA,
                    const void *B, int64_t ldb, int64_t sB, const void *C, int64_t ldc, int64_t sC,
                    int64_t batch, int ab_type, int c_type, bool check_pointers = true) {
    if (transb != 0 && transb != 1) return fail(TDG_INVALID_VALUE, "transb must be 0 or 1");
    if (M < 0 || N < 0 || K < 0 || batch < 0)
        return fail(TDG_INVALID_VALUE, "negative size (M=%lld N=%lld K=%lld batch=%lld)", (long long)M,
                    (long long)N, (long long)K, (long long)batch);
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX)
        return fail(TDG_INVALID_VALUE, "M, N and K must each be below 2^31");
    if (ab_type != TDG_F16 && ab_type != TDG_BF16)
        return fail(TDG_INVALID_VALUE, "ab_type must be TDG_F16 or TDG_BF16");
    if (c_type != TDG_F16 && c_type != TDG_BF16 && c_type != TDG_F32)
        return fail(TDG_INVALID_VALUE, "c_type must be TDG_F16, TDG_BF16 or TDG_F32");
    if (lda < (K > 0 ? K : 1)) return fail(TDG_INVALID_VALUE, "lda (%lld) < K (%lld)", (long long)lda, (long long)K);
    const int64_t bmin = transb ? K : N;
    if (ldb < (bmin > 0 ? bmin : 1))
        return fail(TDG_INVALID_VALUE, "ldb (%lld) < %s (%lld)", (long long)ldb, transb ? "K" : "N", (long long)bmin);
    if (ldc < (N > 0 ? N : 1)) return fail(TDG_INVALID_VALUE, "ldc (%lld) < N (%lld)", (long long)ldc, (long long)N);
    if (sA < 0 || sB < 0 || sC < 0) return fail(TDG_INVALID_VALUE, "negative batch stride");
    if (M == 0 || N == 0 || batch == 0) return TDG_SUCCESS;
    if (check_pointers && C == nullptr) return fail(TDG_INVALID_VALUE, "C is NULL");
    if (check_pointers && K > 0 && (A == nullptr || B == nullptr)) return fail(TDG_INVALID_VALUE, "A or B is NULL");
    if (check_pointers && ((((uintptr_t)A | (uintptr_t)B) & 1u) || ((uintptr_t)C & (c_type == TDG_F32 ? 3u : 1u))))
        return fail(TDG_INVALID_VALUE, "A, B and C must be aligned to their element size");
    if (batch > 1 && sC < (M - 1) * ldc + N)
        return fail(TDG_INVALID_VALUE, "strideC (%lld) lets the C matrices of the batch overlap", (long long)sC);
    const int64_t tiles = cdiv(M, 64) * cdiv(N, 64) * batch;
    if (tiles > (int64_t)INT_MAX) return fail(TDG_INVALID_VALUE, "too many output tiles");
    return TDG_SUCCESS;
}

tdg_status run(int transb, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t sA,
               const void *B, int64_t ldb, int64_t sB, void *C, int64_t ldc, int64_t sC, int64_t batch,
               tdg_dtype ab_type, tdg_dtype c_type, int config, void *stream) {
    g_err[0] = '\0';
    tdg_status st = validate(transb, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, batch, ab_type, c_type);
    if (st != TDG_SUCCESS) return st;
    if (M == 0 || N == 0 || batch == 0) return TDG_SUCCESS;
    const bool vec = vec_ok(transb, N, K, A, lda, sA, B, ldb, sB, batch);
    if (config < -1 || config >= kNumConfigs)
        return fail(TDG_INVALID_VALUE, "config %d out of range [-1, %d)", config, kNumConfigs);
    if (config == -1) config = choose(transb, vec, M, N, batch, lda, ldb, ldc, c_type);
    const Config &cf = kConfigs[config];
    if (cf.vec && !vec)
        return fail(TDG_INVALID_VALUE, "config %s needs 16-byte aligned operands with 8-element granules", cf.name);
    if (!config_ok(cf, transb, vec, lda, ldb, ldc, c_type))
        return fail(TDG_INVALID_VALUE, "config %s cannot serve these leading dimensions or this layout", cf.name);
    st = check_device();
    if (st != TDG_SUCCESS) return st;

    GemmArgs a;
    a.A = static_cast<const uint16_t *>(A);
    a.B = static_cast<const uint16_t *>(B);
    a.C = C;
    a.lda = lda; a.ldb = ldb; a.ldc = ldc;
    a.sA = batch > 1 ? sA : 0;
    a.sB = batch > 1 ? sB : 0;
    a.sC = batch > 1 ? sC : 0;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.tiles_m = (int)cdiv(M, cf.bm);
    a.tiles_n = (int)cdiv(N, cf.bn);
    a.tiles_per_batch = a.tiles_m * a.tiles_n;
    const int64_t grid = (int64_t)a.tiles_per_batch * batch;
    if (grid > (int64_t)INT_MAX) return fail(TDG_INVALID_VALUE, "too many output tiles");

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (transb == 0)
        e = (ab_type == TDG_F16) ? launch_t0_ab0(config, c_type, a, grid, s) : launch_t0_ab1(config, c_type, a, grid, s);
    else
        e = (ab_type == TDG_F16) ? launch_t1_ab0(config, c_type, a, grid, s) : launch_t1_ab1(config, c_type, a, grid, s);
    if (e != hipSuccess) return fail(TDG_LAUNCH_FAILED, "kernel launch failed: %s", hipGetErrorString(e));
    return TDG_SUCCESS;
}

}  // namespace
}  // namespace tdg

extern "C" {

tdg_status tdg_gemm_nn(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                       void *C, int64_t ldc, tdg_dtype ab_type, tdg_dtype c_type, void *stream) {
    return tdg::run(0, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, ab_type, c_type, -1, stream);
}

tdg_status tdg_gemm_tn(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                       void *C, int64_t ldc, tdg_dtype ab_type, tdg_dtype c_type, void *stream) {
    return tdg::run(1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, ab_type, c_type, -1, stream);
}

tdg_status tdg_gemm_nn_batched(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t strideA,
                               const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc,
                               int64_t strideC, int64_t batch, tdg_dtype ab_type, tdg_dtype c_type,
                               void *stream) {
    return tdg::run(0, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type, c_type, -1,
                    stream);
}

tdg_status tdg_gemm_tn_batched(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t strideA,
                               const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc,
                               int64_t strideC, int64_t batch, tdg_dtype ab_type, tdg_dtype c_type,
                               void *stream) {
    return tdg::run(1, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type, c_type, -1,
                    stream);
}

tdg_status tdg_gemm_ex(int transb, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t strideA,
                       const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc, int64_t strideC,
                       int64_t batch, tdg_dtype ab_type, tdg_dtype c_type, int config, void *stream) {
    return tdg::run(transb, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type, c_type,
                    config, stream);
}

int tdg_num_configs(void) { return tdg::kNumConfigs; }

const char *tdg_config_name(int config) {
    if (config < 0 || config >= tdg::kNumConfigs) return nullptr;
    return tdg::kConfigs[config].name;
}

int tdg_select_config(int transb, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                      int64_t ldb, const void *C, int64_t ldc, int64_t batch, tdg_dtype ab_type,
                      tdg_dtype c_type) {
    // Batch strides play no part in the choice except through alignment; take
    // them as granule multiples here.
    if (tdg::validate(transb, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, batch > 1 ? (M - 1) * ldc + N : 0, batch,
                      ab_type, c_type, false) != TDG_SUCCESS)
        return -1;
    const bool vec = tdg::vec_ok(transb, N, K, A, lda, 0, B, ldb, 0, batch);
    return tdg::choose(transb, vec, M, N, batch, lda, ldb, ldc, c_type);
}

const char *tdg_status_string(tdg_status status) {
    switch (status) {
    case TDG_SUCCESS: return "TDG_SUCCESS";
    case TDG_INVALID_VALUE: return "TDG_INVALID_VALUE";
    case TDG_NOT_SUPPORTED: return "TDG_NOT_SUPPORTED";
    case TDG_LAUNCH_FAILED: return "TDG_LAUNCH_FAILED";
    default: return "TDG_UNKNOWN_STATUS";
    }
}

const char *tdg_last_error(void) { return tdg::g_err; }

int tdg_abi_version(void) { return TDG_ABI_VERSION; }

}  // extern "C"
