// tdg_api.cpp -- the C ABI of the tiled dense GEMM library (host side).
//
// Validates arguments, picks a tile configuration and enqueues its kernels
// on the caller's stream: one launch, or two over disjoint parts of C when a
// single problem's 256 x 256 tiles leave a partial last round (plan_retile).
// No allocation, no synchronisation, no per-call state beyond the
// thread-local error text, a per-device architecture check made once and
// the autotuning table.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "../../include/tdg.h"
#include "gemm_common.hpp"

namespace tdg {

hipError_t launch_t0_ab0(int cfg, int ct, int transa, const GemmArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_t0_ab1(int cfg, int ct, int transa, const GemmArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_t1_ab0(int cfg, int ct, int transa, const GemmArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_t1_ab1(int cfg, int ct, int transa, const GemmArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_f8_a0_b0(int cfg, int ct, int bscale, const F8Args &a, int64_t grid, hipStream_t s);
hipError_t launch_f8_a0_b1(int cfg, int ct, int bscale, const F8Args &a, int64_t grid, hipStream_t s);
hipError_t launch_f8_a1_b0(int cfg, int ct, int bscale, const F8Args &a, int64_t grid, hipStream_t s);
hipError_t launch_f8_a1_b1(int cfg, int ct, int bscale, const F8Args &a, int64_t grid, hipStream_t s);

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

// Architecture check and compute-unit count, once per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cus[kMaxDevices];          // compute units (valid once g_arch_state is set)

tdg_status check_device(int *cus = nullptr, int *device = nullptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(TDG_NOT_SUPPORTED, "no HIP device is current");
    if (device) *device = dev;
    if (dev < 0 || dev >= kMaxDevices) return fail(TDG_NOT_SUPPORTED, "device index %d out of range", dev);
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(TDG_NOT_SUPPORTED, "cannot query device %d", dev);
        st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        g_arch_state[dev].store(st, std::memory_order_release);
        if (st != 1) return fail(TDG_NOT_SUPPORTED, "device %d is %s, this library targets gfx950", dev,
                                 prop.gcnArchName);
    }
    if (st != 1) return fail(TDG_NOT_SUPPORTED, "device %d is not gfx950", dev);
    if (cus) *cus = g_cus[dev].load(std::memory_order_relaxed);
    return TDG_SUCCESS;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Whether the vectorised path may serve these operands: 16-byte aligned
// bases, row strides and batch strides that keep every 8-element granule
// aligned, and contiguous extents (K for an A stored M x K or a B stored
// N x K, M for an A stored K x M, N for a B stored K x N) that are whole
// granules.
bool vec_ok(int transa, int transb, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t sA,
            const void *B, int64_t ldb, int64_t sB, int64_t batch) {
    if (!aligned16(A) || !aligned16(B)) return false;
    if ((lda & 7) || (ldb & 7)) return false;
    if ((transa ? M : K) & 7) return false;
    if ((transb ? K : N) & 7) return false;
    if (batch > 1 && ((sA & 7) || (sB & 7))) return false;
    return true;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Whether configuration `cf` can serve the operands: an A stored K x M only
// on the 16 x 16 x 32 kernel; the vectorised kinds need vec_ok; the
// direct-to-LDS kinds also need every in-tile byte offset below 2^31 (buffer
// offsets are 32-bit) and, for an operand stored K-strided (A as K x M, B as
// K x N), rows of at least 16 granules in LDS.
bool config_ok(const Config &cf, int transa, int transb, bool vec, int64_t lda, int64_t ldb, int64_t ldc,
               int c_type) {
    if (transa && cf.kind != 2) return false;        // (the other kinds read A stored M x K only)
    if (!cf.vec) return true;
    if (!vec) return false;
    if (cf.kind < 1) return true;
    const int64_t lim = (int64_t)1 << 31;
    const int64_t es = (c_type == TDG_F32) ? 4 : 2;
    if ((int64_t)cf.bm * ldc * es >= lim) return false;
    if ((transa ? (int64_t)cf.bk : (int64_t)cf.bm) * lda * 2 >= lim) return false;
    if ((transb ? (int64_t)cf.bn : (int64_t)cf.bk) * ldb * 2 >= lim) return false;
    if (!transb && cf.bn / 8 < 16) return false;
    if (transa && cf.bm / 8 < 16) return false;
    return true;
}

// The one-tile 16 x 16 x 32 kernel, plain or with the A window: the kinds
// that take split-K and partial-round schedules.
bool one_tile_m16(const Config &cf) { return cf.kind == 2 || cf.kind == 5; }

int config_by_name(const char *name) {
    for (int i = 0; i < kNumConfigs; ++i)
        if (strcmp(kConfigs[i].name, name) == 0) return i;
    return -1;
}

// Whether A's rows start off the 128-byte lines (A stored M x K, lda not a
// multiple of 64 elements), where the A-window forms pay.  Measured against
// the plain forms (same library, one box, bit-identical): 256 x 256 tiles
// TN 7-8% faster (4096^2 x 3000, 8192^2 x 3000) and NN 1-1.5% (8192^2 x
// 3000, the 4095 x 4096 band of 4095 x 5000 x 3000); 128 x 128 tiles TN 8%
// faster on two shapes but NN 3-6% slower (1024^2 and 2048^2 x 3000), so the
// 128 x 128 form is chosen for TN only (`big` selects the tile size).
bool a_window_pays(int transa, int transb, int64_t lda, bool big) {
    return !transa && (big || transb) && (lda * 2) % 128 != 0;
}

// Split-K schedule for the 16x16x32 kernel (NineToothed primer s4 names the
// alternative to keeping K inside one program: split it, at the price of a
// merge step).  With `cus` workgroups running at once, a problem of fewer
// tiles than that would leave most of the chip idle; each tile is cut
// instead into `split` K slices (at most cus / tiles, each at least
// kMinSliceTiles K tiles), run by separate workgroups and merged by the last
// slice to finish.  The kernel also takes whole tiles before the split
// ones, which serves a partial last round (plan_round_split below).
constexpr int64_t kMinSliceTiles = 16;

struct SplitPlan {
    int64_t dp_tiles;   // whole tiles, one workgroup each
    int64_t sk_tiles;   // split tiles
    int split;          // K slices per split tile (1: no split)
};

SplitPlan plan_split(int64_t tiles, int64_t nk, int64_t cus) {
    SplitPlan pl{tiles, 0, 1};
    if (cus <= 0 || tiles <= 0 || tiles >= cus) return pl;
    const int64_t rem = tiles % cus;
    if (rem == 0) return pl;
    int64_t sp = cus / rem;
    if (sp > nk / kMinSliceTiles) sp = nk / kMinSliceTiles;
    if (sp < 2) return pl;
    pl.dp_tiles = tiles - rem;
    pl.sk_tiles = rem;
    pl.split = (int)sp;
    return pl;
}

// A partial last round in one launch (stream-K style: whole tiles, then the
// tiles of the partial round cut into K slices that fill the chip): more
// 256 x 256 tiles than `cus` but not a whole number of rounds, e.g. 320
// tiles on 256 CUs.  The tiles of whole rounds are whole-tile work items;
// the `rem` tiles left over are each cut into at most cus / rem K slices of
// at least kMinRoundSliceTiles K tiles, merged by the last slice to finish.
// Workgroups that finish their whole tile early start on the slices, so the
// last round is spread over every CU instead of running on rem of them.
constexpr int64_t kMinRoundSliceTiles = 8;

SplitPlan plan_round_split(int64_t tiles, int64_t nk, int64_t cus) {
    SplitPlan pl{tiles, 0, 1};
    if (cus <= 0 || tiles <= cus) return pl;
    const int64_t rem = tiles % cus;
    if (rem == 0) return pl;
    int64_t sp = cus / rem;
    if (sp > nk / kMinRoundSliceTiles) sp = nk / kMinRoundSliceTiles;
    if (sp < 2) return pl;
    pl.dp_tiles = tiles - rem;
    pl.sk_tiles = rem;
    pl.split = (int)sp;
    return pl;
}

// Workspace layout: one int counter per possible split tile (fewer than
// `cus` of them) at the start, padded to 256 bytes, then the fp32 partial
// tiles (split x sk_tiles of them).  The counters sit at the same place
// whatever the sizes of the call, so the zeros one call leaves behind are
// where the next call looks for them.
size_t split_flag_bytes(int64_t cus) { return ((size_t)cus * 4 + 255) / 256 * 256; }
size_t split_ws_bytes(const Config &cf, const SplitPlan &pl, int64_t cus) {
    if (pl.split < 2) return 0;
    return split_flag_bytes(cus) + (size_t)pl.sk_tiles * pl.split * cf.bm * cf.bn * 4;
}

// The largest workspace any call needs on a device with `cus` compute units.
// Only the automatic choice splits K: problems with fewer tiles than CUs on
// 128 x 128 tiles (256 x 256 tiles are chosen only for at least one tile
// per CU), and partial last rounds of 256 x 256 tiles; each plan gives at
// most `cus` slices in all (rem * floor(cus / rem) <= cus).  The first kind
// fits in split_ws_bound_small; a call whose workspace cannot hold the
// second serves the partial round another way (the cut in run()).
size_t split_ws_bound_small(int64_t cus) { return split_flag_bytes(cus) + (size_t)cus * 128 * 128 * 4; }
size_t split_ws_bound(int64_t cus) { return split_flag_bytes(cus) + (size_t)cus * 256 * 256 * 4; }

// Whether a split schedule is worth taking for a problem below one round of
// 256 x 256 tiles: it must give at least half the chip a work item.
bool split_pays(const SplitPlan &pl, int64_t cus) {
    return pl.split >= 2 && pl.sk_tiles * pl.split * 2 >= cus;
}

// Tile-configuration choice (measured on MI355X), with `cus` the device's
// compute units: 256 x 256 tiles on the 16 x 16 x 32 MFMA kernel when the
// problem has at least one such tile per CU (its persistent form for
// problems of several rounds with a short K); 128 x 128 tiles on the same
// kernel (8 waves, 4 stages) for smaller problems; the 32 x 32 x 16 direct
// load kernel or the register-staged kernel when the 16 x 16 x 32 kernel
// cannot address the operands; the predicated kernel for misaligned
// operands.
// An A stored K x M (transa) has only the 16 x 16 x 32 kernel: -1 when that
// kernel cannot serve the operands.
int choose(int transa, int transb, bool vec, int64_t M, int64_t N, int64_t K, int64_t batch, int64_t lda,
           int64_t ldb, int64_t ldc, int c_type, int64_t cus) {
    const int64_t b = batch < 1 ? 1 : batch;
    if (vec) {
        const int64_t tiles256 = cdiv(M, 256) * cdiv(N, 256) * b;
        // several rounds with K <= 512 (at most 8 K tiles per output tile):
        // the persistent form, whose next tile's loads and MFMAs overlap the
        // current tile's stores.  16-bit output: 4-22% faster than the
        // one-tile kernel over batches of 1024^2 to 8192^2 products at
        // K = 128..512, both layouts (even at 1024, 1-12% slower from 2048
        // on, where the one-tile kernel's wave priority and simpler loop
        // win).  fp32 output: 2-23% faster on every batched shape measured
        // (32 x 2048^2, 16 x 2048^2, 128 x 1024^2, 8 x 4096^2, 4 x 4096^2),
        // but 6-13% slower on a single 8192^2 product, so only for batches.
        // Not in a single round.
        const int pid = config_by_name("256x256x64_s2_w2x4_m16p");
        const bool persist_ok = c_type != TDG_F32 || b >= 2;
        if (tiles256 >= 2 * cus && K > 0 && K <= 512 && persist_ok && !transa &&
            config_ok(kConfigs[pid], transa, transb, vec, lda, ldb, ldc, c_type))
            return pid;
        // one round or more, TN with A rows off the 128-byte lines: the
        // A-window form, which loads each row as aligned 128-byte chunks (the
        // kernel works out every row's shift from the actual addresses, so
        // this is only the choice; a_window_pays has the measurements)
        const int aw = config_by_name("256x256x64_s2_w2x4_m16aw");
        if (tiles256 >= cus && a_window_pays(transa, transb, lda, true) &&
            config_ok(kConfigs[aw], transa, transb, vec, lda, ldb, ldc, c_type))
            return aw;
        const int id = config_by_name("256x256x64_s2_w2x4_m16");
        if (tiles256 >= cus && config_ok(kConfigs[id], transa, transb, vec, lda, ldb, ldc, c_type)) return id;
        const int mid_aw = config_by_name("128x128x64_s4_w2x4_m16aw");
        if (a_window_pays(transa, transb, lda, false) && config_ok(kConfigs[mid_aw], transa, transb, vec, lda, ldb, ldc, c_type))
            return mid_aw;
        const int mid = config_by_name("128x128x64_s4_w2x4_m16");
        if (config_ok(kConfigs[mid], transa, transb, vec, lda, ldb, ldc, c_type)) return mid;
        if (transa) return -1;
        const int small = config_by_name("128x128x64_s2_w2x2_lds");
        if (config_ok(kConfigs[small], transa, transb, vec, lda, ldb, ldc, c_type)) return small;
        return config_by_name((cdiv(M, 128) * cdiv(N, 128) * b >= 256) ? "128x128x64_w2x2_vec" : "64x64x64_w2x2_vec");
    }
    if (transa) return -1;
    return config_by_name((cdiv(M, 128) * cdiv(N, 128) * b >= 256) ? "128x128x64_w2x2_pred" : "64x64x64_w2x2_pred");
}

// Argument checks in the caller's terms: A stored M x K (transa 0) or K x M
// (transa 1), B stored K x N (transb 0) or N x K (transb 1), C stored M x N
// (transc 0) or N x M (transc 1).
tdg_status validate(int transa, int transb, int transc, int64_t M, int64_t N, int64_t K, const void *A,
                    int64_t lda, int64_t sA, const void *B, int64_t ldb, int64_t sB, const void *C, int64_t ldc,
                    int64_t sC, int64_t batch, int ab_type, int c_type, bool check_pointers = true) {
    if (transa != 0 && transa != 1) return fail(TDG_INVALID_VALUE, "transa must be 0 or 1");
    if (transb != 0 && transb != 1) return fail(TDG_INVALID_VALUE, "transb must be 0 or 1");
    if (transc != 0 && transc != 1) return fail(TDG_INVALID_VALUE, "transc must be 0 or 1");
    if (M < 0 || N < 0 || K < 0 || batch < 0)
        return fail(TDG_INVALID_VALUE, "negative size (M=%lld N=%lld K=%lld batch=%lld)", (long long)M,
                    (long long)N, (long long)K, (long long)batch);
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX)
        return fail(TDG_INVALID_VALUE, "M, N and K must each be below 2^31");
    if (ab_type != TDG_F16 && ab_type != TDG_BF16)
        return fail(TDG_INVALID_VALUE, "ab_type must be TDG_F16 or TDG_BF16");
    if (c_type != TDG_F16 && c_type != TDG_BF16 && c_type != TDG_F32)
        return fail(TDG_INVALID_VALUE, "c_type must be TDG_F16, TDG_BF16 or TDG_F32");
    const int64_t amin = transa ? M : K, bmin = transb ? K : N, cmin = transc ? M : N;
    if (lda < (amin > 0 ? amin : 1))
        return fail(TDG_INVALID_VALUE, "lda (%lld) < %s (%lld)", (long long)lda, transa ? "M" : "K", (long long)amin);
    if (ldb < (bmin > 0 ? bmin : 1))
        return fail(TDG_INVALID_VALUE, "ldb (%lld) < %s (%lld)", (long long)ldb, transb ? "K" : "N", (long long)bmin);
    if (ldc < (cmin > 0 ? cmin : 1))
        return fail(TDG_INVALID_VALUE, "ldc (%lld) < %s (%lld)", (long long)ldc, transc ? "M" : "N", (long long)cmin);
    if (sA < 0 || sB < 0 || sC < 0) return fail(TDG_INVALID_VALUE, "negative batch stride");
    if (M == 0 || N == 0 || batch == 0) return TDG_SUCCESS;
    if (check_pointers && C == nullptr) return fail(TDG_INVALID_VALUE, "C is NULL");
    if (check_pointers && K > 0 && (A == nullptr || B == nullptr)) return fail(TDG_INVALID_VALUE, "A or B is NULL");
    if (check_pointers && ((((uintptr_t)A | (uintptr_t)B) & 1u) || ((uintptr_t)C & (c_type == TDG_F32 ? 3u : 1u))))
        return fail(TDG_INVALID_VALUE, "A, B and C must be aligned to their element size");
    if (batch > 1 && sC < (transc ? (N - 1) * ldc + M : (M - 1) * ldc + N))
        return fail(TDG_INVALID_VALUE, "strideC (%lld) lets the C matrices of the batch overlap", (long long)sC);
    const int64_t tiles = cdiv(M, 64) * cdiv(N, 64) * batch;
    if (tiles > (int64_t)INT_MAX) return fail(TDG_INVALID_VALUE, "too many output tiles");
    return TDG_SUCCESS;
}

// One launch of configuration `config` over a whole (sub-)problem.
tdg_status launch(int config, int transa, int transb, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                  int64_t sA,
                  const void *B, int64_t ldb, int64_t sB, void *C, int64_t ldc, int64_t sC, int64_t batch,
                  tdg_dtype ab_type, tdg_dtype c_type, void *stream, void *ws, size_t ws_bytes, int cus,
                  const SplitPlan *plan = nullptr) {
    const Config &cf = kConfigs[config];
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
    const int64_t tiles = (int64_t)a.tiles_per_batch * batch;
    if (cf.kind == 3) {
        // persistent: one workgroup per CU (its LDS stages take most of a CU),
        // each walking tiles w, w + grid, ...; a K of 0 (nothing to walk) is
        // served by the one-tile-per-workgroup kernel of the same tiles
        if (K == 0)
            return launch(config_by_name("256x256x64_s2_w2x4_m16"), transa, transb, M, N, K, A, lda, sA, B, ldb, sB, C,
                          ldc, sC, batch, ab_type, c_type, stream, nullptr, 0, cus);
        a.ws = nullptr;
        a.ws_flags = nullptr;
        a.dp_tiles = (int)tiles;
        a.sk_split = 1;
        const int64_t grid = tiles < cus ? tiles : cus;
        hipStream_t s = static_cast<hipStream_t>(stream);
        hipError_t e;
        if (transb == 0)
            e = (ab_type == TDG_F16) ? launch_t0_ab0(config, c_type, transa, a, grid, s)
                                     : launch_t0_ab1(config, c_type, transa, a, grid, s);
        else
            e = (ab_type == TDG_F16) ? launch_t1_ab0(config, c_type, transa, a, grid, s)
                                     : launch_t1_ab1(config, c_type, transa, a, grid, s);
        if (e != hipSuccess) return fail(TDG_LAUNCH_FAILED, "kernel launch failed: %s", hipGetErrorString(e));
        return TDG_SUCCESS;
    }
    SplitPlan pl{tiles, 0, 1};
    if (plan != nullptr) {
        pl = *plan;
    } else if (one_tile_m16(cf) && ws != nullptr) {
        pl = plan_split(tiles, cdiv(K, cf.bk), cus);
        if (!split_pays(pl, cus)) pl = SplitPlan{tiles, 0, 1};
    }
    const size_t need = split_ws_bytes(cf, pl, cus);
    if (need > ws_bytes)
        return fail(TDG_INVALID_VALUE, "workspace of %zu bytes is smaller than the %zu bytes this call needs", ws_bytes,
                    need);
    const bool split = pl.split >= 2;
    a.ws_flags = split ? static_cast<int *>(ws) : nullptr;
    a.ws = split ? reinterpret_cast<float *>(static_cast<char *>(ws) + split_flag_bytes(cus)) : nullptr;
    a.dp_tiles = (int)pl.dp_tiles;
    a.sk_split = pl.split;
    const int64_t grid = pl.dp_tiles + pl.sk_tiles * pl.split;
    if (grid > (int64_t)INT_MAX) return fail(TDG_INVALID_VALUE, "too many output tiles");

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (transb == 0)
        e = (ab_type == TDG_F16) ? launch_t0_ab0(config, c_type, transa, a, grid, s)
                                 : launch_t0_ab1(config, c_type, transa, a, grid, s);
    else
        e = (ab_type == TDG_F16) ? launch_t1_ab0(config, c_type, transa, a, grid, s)
                                 : launch_t1_ab1(config, c_type, transa, a, grid, s);
    if (e != hipSuccess) return fail(TDG_LAUNCH_FAILED, "kernel launch failed: %s", hipGetErrorString(e));
    return TDG_SUCCESS;
}

int64_t gcd64(int64_t a, int64_t b) {
    while (b) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

// Wave quantisation without a merge step: when a single problem has more
// 256 x 256 tiles than `cus` but not a whole number of rounds, the output is
// cut into a part that holds whole rounds of 256 x 256 tiles (a band of tile
// columns, or of tile rows) and the rest, which is covered by 128 x 128
// tiles, four times as many work items for the same area.  Cost model in
// units of one 256 x 256 tile's time: a 128 x 128 tile takes 0.4 of it
// (a quarter of the work at a lower rate).  Returns the cut (a multiple of
// 256, in columns if *cols else in rows) or 0 when cutting does not pay.
int64_t plan_retile(int64_t M, int64_t N, int64_t cus, bool *cols) {
    const int64_t tm = cdiv(M, 256), tn = cdiv(N, 256), tiles = tm * tn;
    if (cus <= 0 || tiles <= cus || tiles % cus == 0) return 0;
    double best = (double)cdiv(tiles, cus) * 0.9;
    int64_t cut = 0;
    for (int pass = 0; pass < 2; ++pass) {
        const int64_t mine = pass == 0 ? tm : tn, other = pass == 0 ? tn : tm;
        const int64_t step = cus / gcd64(mine, cus);          // tile lines per whole round
        const int64_t lines = (other - 1) / step * step;      // keep a remainder
        if (lines <= 0) continue;
        const int64_t rest = pass == 0 ? cdiv(M, 128) * cdiv(N - 256 * lines, 128)
                                       : cdiv(M - 256 * lines, 128) * cdiv(N, 128);
        double rem_cost = 0.4 * (double)rest / (double)cus;
        if (rem_cost < 0.4) rem_cost = 0.4;
        const double cost = (double)(mine * lines / cus) + rem_cost;
        if (cost < best) {
            best = cost;
            cut = 256 * lines;
            *cols = pass == 0;
        }
    }
    return cut;
}

// Autotuning results: for a problem (device, storage orders, sizes, types
// and whether the operands can take the vectorised kernels), the
// configuration measured fastest by tdg_autotune, or -1 when the automatic
// schedule won.
struct TuneKey {
    int dev, transa, transb, transc, ab, ct, vec;
    int64_t M, N, K, batch;
    bool operator<(const TuneKey &o) const {
        return std::tie(dev, transa, transb, transc, ab, ct, vec, M, N, K, batch) <
               std::tie(o.dev, o.transa, o.transb, o.transc, o.ab, o.ct, o.vec, o.M, o.N, o.K, o.batch);
    }
};
std::mutex g_tune_mu;
std::map<TuneKey, int> g_tune;

// The tuned configuration for `k`, or -2 when the problem was not tuned.
int tuned_config(const TuneKey &k) {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    const auto it = g_tune.find(k);
    return it == g_tune.end() ? -2 : it->second;
}

// C = op(A) * op(B) (A stored M x K or K x M, B stored K x N or N x K),
// written as C or as C^T.  A transposed store is the product with the
// operands exchanged, C^T = B^T A^T: (transa, transb, transc = 1) on (A, B)
// runs as (!transb, !transa, 0) on (B, A) with M and N exchanged.
// An automatic call (config -1) of a tuned problem takes the tuned
// configuration (use_tuned false: the library's own choice, for tuning).
tdg_status run(int transa, int transb, int transc, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
               int64_t sA, const void *B, int64_t ldb, int64_t sB, void *C, int64_t ldc, int64_t sC, int64_t batch,
               tdg_dtype ab_type, tdg_dtype c_type, int config, void *stream, void *ws = nullptr,
               size_t ws_bytes = 0, bool use_tuned = true) {
    g_err[0] = '\0';
    tdg_status st = validate(transa, transb, transc, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, batch, ab_type,
                             c_type);
    if (st != TDG_SUCCESS) return st;
    if (M == 0 || N == 0 || batch == 0) return TDG_SUCCESS;
    const int ta_in = transa, tb_in = transb, tc_in = transc;
    const int64_t M_in = M, N_in = N;
    if (transc) {
        const int ta = !transb, tb = !transa;
        transa = ta;
        transb = tb;
        transc = 0;
        std::swap(M, N);
        std::swap(A, B);
        std::swap(lda, ldb);
        std::swap(sA, sB);
    }
    const bool vec = vec_ok(transa, transb, M, N, K, A, lda, sA, B, ldb, sB, batch);
    if (config < -1 || config >= kNumConfigs)
        return fail(TDG_INVALID_VALUE, "config %d out of range [-1, %d)", config, kNumConfigs);
    if (ws != nullptr && ((uintptr_t)ws & 255u))
        return fail(TDG_INVALID_VALUE, "workspace must be 256-byte aligned");
    const bool automatic = config == -1;
    if (!automatic) {
        const Config &forced = kConfigs[config];
        if (forced.vec && !vec)
            return fail(TDG_INVALID_VALUE, "config %s needs 16-byte aligned operands with 8-element granules",
                        forced.name);
        if (!config_ok(forced, transa, transb, vec, lda, ldb, ldc, c_type))
            return fail(TDG_INVALID_VALUE, "config %s cannot serve these leading dimensions or this layout",
                        forced.name);
    }
    int cus = 0, dev = 0;
    st = check_device(&cus, &dev);
    if (st != TDG_SUCCESS) return st;
    bool tuned = false;
    if (automatic && use_tuned) {
        const int t = tuned_config(TuneKey{dev, ta_in, tb_in, tc_in, ab_type, c_type, vec ? 1 : 0, M_in, N_in, K, batch});
        if (t >= 0 && config_ok(kConfigs[t], transa, transb, vec, lda, ldb, ldc, c_type)) {
            config = t;
            tuned = true;
        }
    }
    if (automatic && !tuned) config = choose(transa, transb, vec, M, N, K, batch, lda, ldb, ldc, c_type, cus);
    if (config < 0)
        return fail(TDG_NOT_SUPPORTED,
                    "layout transa=%d transb=%d transc=%d runs on the vectorised kernel only: 16-byte aligned A and B, "
                    "leading dimensions, batch strides and contiguous extents multiples of 8 elements",
                    ta_in, tb_in, tc_in);
    const Config &cf = kConfigs[config];

    // Automatic choice on a single problem with a partial last round of
    // 256 x 256 tiles: whole rounds on one band of C and 128 x 128 tiles on
    // the rest (two launches on the stream, disjoint parts of C), or one
    // launch whose last round is cut into K slices (plan_round_split), when
    // the workspace holds their partial tiles and either no band of whole
    // rounds exists or the 128 x 128 rest would keep fewer than half of the
    // CUs busy.  Measured on MI355X (one launch / two launches): 0.71 and
    // 0.85 with no band (17 x 17 tiles, K 16384 and 4096), 0.85 with a rest
    // of 64 small tiles (K 32768), 0.98 with a rest of 128, 1.03 and 1.13
    // with rests of 128 and 256 (4095 x 5000 x 3000): the merge of 256 x 256
    // partial tiles costs more than a well-filled rest round.
    if (automatic && !tuned && one_tile_m16(cf) && batch == 1 && ws != nullptr) {
        const SplitPlan rp = plan_round_split(cdiv(M, cf.bm) * cdiv(N, cf.bn), cdiv(K, cf.bk), cus);
        if (rp.split >= 2 && split_ws_bytes(cf, rp, cus) <= ws_bytes) {
            bool cols = true;
            const int64_t cut = plan_retile(M, N, cus, &cols);
            const int64_t rest = cut == 0 ? 0
                                 : (cols ? cdiv(M, 128) * cdiv(N - cut, 128) : cdiv(M - cut, 128) * cdiv(N, 128));
            if (cut == 0 || rest * 2 < cus)
                return launch(config, transa, transb, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, batch, ab_type,
                              c_type, stream, ws, ws_bytes, cus, &rp);
        }
    }
    if (automatic && !tuned && cf.kind >= 2 && batch == 1) {
        const int small = config_by_name(a_window_pays(transa, transb, lda, false) ? "128x128x64_s4_w2x4_m16aw"
                                                                            : "128x128x64_s4_w2x4_m16");
        bool cols = true;
        const int64_t cut = plan_retile(M, N, cus, &cols);
        if (cut > 0 && config_ok(kConfigs[small], transa, transb, vec, lda, ldb, ldc, c_type)) {
            const int64_t es = (c_type == TDG_F32) ? 4 : 2;
            const uint16_t *b16 = static_cast<const uint16_t *>(B);
            const uint16_t *a16 = static_cast<const uint16_t *>(A);
            char *c8 = static_cast<char *>(C);
            if (cols) {
                st = launch(config, transa, transb, M, cut, K, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, ab_type, c_type,
                            stream, nullptr, 0, cus);
                if (st != TDG_SUCCESS) return st;
                return launch(small, transa, transb, M, N - cut, K, A, lda, 0, transb ? b16 + cut * ldb : b16 + cut,
                              ldb, 0, c8 + cut * es, ldc, 0, 1, ab_type, c_type, stream, nullptr, 0, cus);
            }
            st = launch(config, transa, transb, cut, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, ab_type, c_type,
                        stream, nullptr, 0, cus);
            if (st != TDG_SUCCESS) return st;
            return launch(small, transa, transb, M - cut, N, K, transa ? a16 + cut : a16 + cut * lda, lda, 0, B, ldb,
                          0, c8 + cut * ldc * es, ldc, 0, 1, ab_type, c_type, stream, nullptr, 0, cus);
        }
    }
    // (a tuned configuration runs as it was timed: without split-K)
    return launch(config, transa, transb, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, batch, ab_type, c_type,
                  stream, tuned ? nullptr : ws, tuned ? 0 : ws_bytes, cus);
}

// ---- 8-bit operands ----

struct F8Config {
    int bm, bn, stages, wm, wn;
    const char *name;
};

const F8Config kF8Configs[] = {
#define TDG_F8_ROW(ID, BM, BN, ST, WM, WN, NAME) {BM, BN, ST, WM, WN, NAME},
    TDG_F8_CONFIG_LIST(TDG_F8_ROW)
#undef TDG_F8_ROW
};
constexpr int kNumF8Configs = (int)(sizeof(kF8Configs) / sizeof(kF8Configs[0]));

constexpr int kF8ConfigIds[] = {
#define TDG_F8_ID(ID, BM, BN, ST, WM, WN, NAME) ID,
    TDG_F8_CONFIG_LIST(TDG_F8_ID)
#undef TDG_F8_ID
};
constexpr bool f8_ids_in_order(int i) {
    return i == kNumF8Configs || (kF8ConfigIds[i] == i && f8_ids_in_order(i + 1));
}
static_assert(f8_ids_in_order(0), "8-bit configuration ids must be 0, 1, ... in list order");

bool is_f8(int t) { return t == TDG_E4M3 || t == TDG_E5M2; }

// C = sa * sb * blockscaled(A * B^T), written as C or C^T (see tdg.h).
// Every argument check comes before the device check, so that argument
// errors read the same on any host.
tdg_status run_f8(int transc, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int a_type, const void *B,
                  int64_t ldb, int b_type, const void *xa, int64_t ldxa, const void *xb, int64_t ldxb,
                  const float *sa, int64_t inc_sa, const float *sb, int64_t inc_sb, void *C, int64_t ldc,
                  int c_type, int config, void *stream) {
    g_err[0] = '\0';
    if (transc != 0 && transc != 1) return fail(TDG_INVALID_VALUE, "transc must be 0 or 1");
    if (M < 0 || N < 0 || K < 0)
        return fail(TDG_INVALID_VALUE, "negative size (M=%lld N=%lld K=%lld)", (long long)M, (long long)N,
                    (long long)K);
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX) return fail(TDG_INVALID_VALUE, "M, N and K must each be below 2^31");
    if (!is_f8(a_type) || !is_f8(b_type)) return fail(TDG_INVALID_VALUE, "a_type and b_type must be TDG_E4M3 or TDG_E5M2");
    if (c_type != TDG_F16 && c_type != TDG_BF16 && c_type != TDG_F32)
        return fail(TDG_INVALID_VALUE, "c_type must be TDG_F16, TDG_BF16 or TDG_F32");
    const int64_t kmin = K > 0 ? K : 1, cmin = (transc ? M : N) > 0 ? (transc ? M : N) : 1;
    const int64_t nkb = (K + 31) / 32, bmin = nkb > 0 ? nkb : 1;
    if (lda < kmin || ldb < kmin) return fail(TDG_INVALID_VALUE, "lda and ldb must be at least K (%lld)", (long long)K);
    if (ldc < cmin)
        return fail(TDG_INVALID_VALUE, "ldc (%lld) < %s (%lld)", (long long)ldc, transc ? "M" : "N", (long long)cmin);
    if ((xa && ldxa < bmin) || (xb && ldxb < bmin))
        return fail(TDG_INVALID_VALUE, "block-scale row strides must be at least ceil(K/32) = %lld", (long long)nkb);
    if (inc_sa < 0 || inc_sb < 0) return fail(TDG_INVALID_VALUE, "row-scale increments must be nonnegative");
    if (config < -1 || config >= kNumF8Configs)
        return fail(TDG_INVALID_VALUE, "config %d out of range [-1, %d)", config, kNumF8Configs);
    if (M == 0 || N == 0) return TDG_SUCCESS;
    if (C == nullptr) return fail(TDG_INVALID_VALUE, "C is NULL");
    if (K > 0 && (A == nullptr || B == nullptr)) return fail(TDG_INVALID_VALUE, "A or B is NULL");
    if ((uintptr_t)C & (c_type == TDG_F32 ? 3u : 1u)) return fail(TDG_INVALID_VALUE, "C must be aligned to its element size");
    if (((uintptr_t)sa | (uintptr_t)sb) & 3u) return fail(TDG_INVALID_VALUE, "row scales must be 4-byte aligned");
    if (K > 0 && (!aligned16(A) || !aligned16(B) || (lda & 15) || (ldb & 15) || (K & 15)))
        return fail(TDG_NOT_SUPPORTED,
                    "8-bit operands need 16-byte aligned A and B, lda, ldb and K multiples of 16");
    if ((xa && (!aligned16(xa) || (ldxa & 15))) || (xb && (!aligned16(xb) || (ldxb & 15))))
        return fail(TDG_NOT_SUPPORTED, "block-scale arrays need 16-byte aligned bases and row strides multiple of 16");
    // 32-bit buffer offsets inside one tile (at most 256 rows of each array)
    const int64_t lim = (int64_t)1 << 31, es = (c_type == TDG_F32) ? 4 : 2;
    if (256 * lda >= lim || 256 * ldb >= lim || 256 * ldc * es >= lim || 256 * ldxa >= lim || 256 * ldxb >= lim)
        return fail(TDG_NOT_SUPPORTED, "a leading dimension is too large for 32-bit in-tile offsets");
    if (cdiv(M, 128) * cdiv(N, 128) > (int64_t)INT_MAX) return fail(TDG_INVALID_VALUE, "too many output tiles");
    int cus = 0;
    tdg_status st = check_device(&cus);
    if (st != TDG_SUCCESS) return st;
    if (transc) {   // C^T = B * A^T: exchange the operands with their scales
        std::swap(M, N);
        std::swap(A, B);
        std::swap(lda, ldb);
        std::swap(a_type, b_type);
        std::swap(xa, xb);
        std::swap(ldxa, ldxb);
        std::swap(sa, sb);
        std::swap(inc_sa, inc_sb);
    }
    if (config < 0) config = (cdiv(M, 256) * cdiv(N, 256) >= cus) ? 0 : 1;
    const F8Config &cf = kF8Configs[config];
    F8Args a;
    a.A = static_cast<const uint8_t *>(A);
    a.B = static_cast<const uint8_t *>(B);
    a.C = C;
    a.lda = lda; a.ldb = ldb; a.ldc = ldc;
    a.xa = static_cast<const uint8_t *>(xa);
    a.xb = static_cast<const uint8_t *>(xb);
    a.ldxa = ldxa; a.ldxb = ldxb;
    a.sa = sa; a.sb = sb;
    a.inc_sa = inc_sa; a.inc_sb = inc_sb;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.tiles_m = (int)cdiv(M, cf.bm);
    a.tiles_n = (int)cdiv(N, cf.bn);
    a.tiles_per_batch = a.tiles_m * a.tiles_n;
    const int64_t grid = a.tiles_per_batch;
    const int bscale = (xa != nullptr || xb != nullptr) ? 1 : 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int fa = a_type == TDG_E5M2, fb = b_type == TDG_E5M2;
    hipError_t e;
    if (fa == 0)
        e = fb == 0 ? launch_f8_a0_b0(config, c_type, bscale, a, grid, s) : launch_f8_a0_b1(config, c_type, bscale, a, grid, s);
    else
        e = fb == 0 ? launch_f8_a1_b0(config, c_type, bscale, a, grid, s) : launch_f8_a1_b1(config, c_type, bscale, a, grid, s);
    if (e != hipSuccess) return fail(TDG_LAUNCH_FAILED, "kernel launch failed: %s", hipGetErrorString(e));
    return TDG_SUCCESS;
}

// ---- allocation-free calls: a fixed split-K scratch area per GPU ----
//
// The split-K workspace of tdg_gemm_noalloc: one array per GPU, part of the
// library's device code, so it exists from the library's load until the
// process ends and no call allocates.  Host code never uses the array's name
// as an address (on the host it is only a stand-in for the device symbol):
// the address on each device comes from hipGetSymbolAddress, once per device,
// with that device current.  Layout as any workspace: the arrival counters
// first (zero between calls: the loader zero-fills the array and every
// merging slice puts its counter back), then the fp32 partial tiles.
constexpr size_t kScratchBytes = TDG_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (nullptr: not looked up yet)

// The scratch array's address on the current device `dev`.
tdg_status scratch_of(int dev, void **out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(TDG_LAUNCH_FAILED, "cannot find the scratch array on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return TDG_SUCCESS;
}

}  // namespace
}  // namespace tdg

extern "C" {

tdg_status tdg_gemm_noalloc(int transa, int transb, int transc, int64_t M, int64_t N, int64_t K, const void *A,
                            int64_t lda, int64_t strideA, const void *B, int64_t ldb, int64_t strideB, void *C,
                            int64_t ldc, int64_t strideC, int64_t batch, tdg_dtype ab_type, tdg_dtype c_type,
                            void *stream) {
    using namespace tdg;
    g_err[0] = '\0';
    tdg_status st = validate(transa, transb, transc, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                             batch, ab_type, c_type);
    if (st != TDG_SUCCESS) return st;
    if (M == 0 || N == 0 || batch == 0) return TDG_SUCCESS;
    int cus = 0, dev = 0;
    st = check_device(&cus, &dev);
    if (st != TDG_SUCCESS) return st;
    if (split_ws_bound_small(cus) > kScratchBytes)
        return fail(TDG_INVALID_VALUE,
                    "the split-K schedule of a %d-CU device may need %zu bytes, more than the %zu-byte scratch array",
                    cus, split_ws_bound_small(cus), kScratchBytes);
    void *ws = nullptr;
    st = scratch_of(dev, &ws);
    if (st != TDG_SUCCESS) return st;
    return run(transa, transb, transc, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type,
               c_type, -1, stream, ws, kScratchBytes);
}

tdg_status tdg_gemm_f8(int transc, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, tdg_dtype a_type,
                       const void *B, int64_t ldb, tdg_dtype b_type, const void *block_scale_a, int64_t ld_bsa,
                       const void *block_scale_b, int64_t ld_bsb, const float *scale_a, int64_t inc_a,
                       const float *scale_b, int64_t inc_b, void *C, int64_t ldc, tdg_dtype c_type, int config,
                       void *stream) {
    return tdg::run_f8(transc, M, N, K, A, lda, a_type, B, ldb, b_type, block_scale_a, ld_bsa, block_scale_b, ld_bsb,
                       scale_a, inc_a, scale_b, inc_b, C, ldc, c_type, config, stream);
}

int tdg_f8_num_configs(void) { return tdg::kNumF8Configs; }

const char *tdg_f8_config_name(int config) {
    if (config < 0 || config >= tdg::kNumF8Configs) return nullptr;
    return tdg::kF8Configs[config].name;
}

tdg_status tdg_gemm_nn(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                       void *C, int64_t ldc, tdg_dtype ab_type, tdg_dtype c_type, void *stream) {
    return tdg::run(0, 0, 0, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, ab_type, c_type, -1, stream);
}

tdg_status tdg_gemm_tn(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                       void *C, int64_t ldc, tdg_dtype ab_type, tdg_dtype c_type, void *stream) {
    return tdg::run(0, 1, 0, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, ab_type, c_type, -1, stream);
}

tdg_status tdg_gemm_nn_batched(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t strideA,
                               const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc,
                               int64_t strideC, int64_t batch, tdg_dtype ab_type, tdg_dtype c_type,
                               void *stream) {
    return tdg::run(0, 0, 0, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type, c_type, -1,
                    stream);
}

tdg_status tdg_gemm_tn_batched(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t strideA,
                               const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc,
                               int64_t strideC, int64_t batch, tdg_dtype ab_type, tdg_dtype c_type,
                               void *stream) {
    return tdg::run(0, 1, 0, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type, c_type, -1,
                    stream);
}

tdg_status tdg_gemm_ws(int transb, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t strideA,
                       const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc, int64_t strideC,
                       int64_t batch, tdg_dtype ab_type, tdg_dtype c_type, void *workspace, size_t workspace_bytes,
                       void *stream) {
    return tdg::run(0, transb, 0, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type, c_type,
                    -1, stream, workspace, workspace_bytes);
}

tdg_status tdg_gemm(int transa, int transb, int transc, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                    int64_t strideA, const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc,
                    int64_t strideC, int64_t batch, tdg_dtype ab_type, tdg_dtype c_type, void *workspace,
                    size_t workspace_bytes, void *stream) {
    return tdg::run(transa, transb, transc, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch,
                    ab_type, c_type, -1, stream, workspace, workspace_bytes);
}

size_t tdg_gemm_workspace_size(int transb, int64_t M, int64_t N, int64_t K, int64_t batch, int num_cus) {
    if (M <= 0 || N <= 0 || K <= 0 || batch <= 0 || (transb != 0 && transb != 1)) return 0;
    int cus = num_cus;
    if (cus <= 0 && tdg::check_device(&cus) != TDG_SUCCESS) return 0;
    // the configuration the library picks for vectorisable operands
    const int id = tdg::choose(0, transb, true, M, N, K, batch, K, transb ? K : N, N, TDG_F32, cus);
    if (id < 0) return 0;
    const tdg::Config &cf = tdg::kConfigs[id];
    if (!tdg::one_tile_m16(cf)) return 0;
    const int64_t tiles = tdg::cdiv(M, cf.bm) * tdg::cdiv(N, cf.bn) * batch;
    if (batch == 1 && tiles > cus) {
        // (an upper bound: run() may serve the problem with the cut instead)
        const tdg::SplitPlan rp = tdg::plan_round_split(tiles, tdg::cdiv(K, cf.bk), cus);
        return rp.split >= 2 ? tdg::split_ws_bytes(cf, rp, cus) : 0;
    }
    const tdg::SplitPlan pl = tdg::plan_split(tiles, tdg::cdiv(K, cf.bk), cus);
    if (!tdg::split_pays(pl, cus)) return 0;
    return tdg::split_ws_bytes(cf, pl, cus);
}

size_t tdg_gemm_workspace_bound(int num_cus) {
    int cus = num_cus;
    if (cus <= 0 && tdg::check_device(&cus) != TDG_SUCCESS) return 0;
    return tdg::split_ws_bound(cus);
}

tdg_status tdg_gemm_ex(int transb, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t strideA,
                       const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc, int64_t strideC,
                       int64_t batch, tdg_dtype ab_type, tdg_dtype c_type, int config, void *stream) {
    return tdg::run(0, transb, 0, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, ab_type, c_type,
                    config, stream);
}

tdg_status tdg_autotune(int transa, int transb, int transc, int64_t M, int64_t N, int64_t K, const void *A,
                        int64_t lda, int64_t strideA, const void *B, int64_t ldb, int64_t strideB, void *C,
                        int64_t ldc, int64_t strideC, int64_t batch, tdg_dtype ab_type, tdg_dtype c_type,
                        void *workspace, size_t workspace_bytes, int reps, int *best_config, void *stream) {
    using namespace tdg;
    g_err[0] = '\0';
    if (reps < 1 || reps > 1000) return fail(TDG_INVALID_VALUE, "reps must be in [1, 1000]");
    tdg_status st = validate(transa, transb, transc, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                             batch, ab_type, c_type);
    if (st != TDG_SUCCESS) return st;
    int cus = 0, dev = 0;
    st = check_device(&cus, &dev);
    if (st != TDG_SUCCESS) return st;
    if (M == 0 || N == 0 || batch == 0 || K == 0) {
        if (best_config) *best_config = -1;
        return TDG_SUCCESS;
    }
    // the candidates in the library's own terms (a transposed store runs as
    // the exchanged product)
    const int ta = transc ? !transb : transa, tb = transc ? !transa : transb;
    const void *iA = transc ? B : A, *iB = transc ? A : B;
    const int64_t iM = transc ? N : M, iN = transc ? M : N, ilda = transc ? ldb : lda, ildb = transc ? lda : ldb;
    const int64_t isA = transc ? strideB : strideA, isB = transc ? strideA : strideB;
    const bool vec = vec_ok(ta, tb, iM, iN, K, iA, ilda, isA, iB, ildb, isB, batch);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        return fail(TDG_LAUNCH_FAILED, "cannot create timing events");
    }
    int best = -2;
    float best_ms = 0.0f;
    for (int cand = -1; cand < kNumConfigs; ++cand) {
        if (cand >= 0 && ((kConfigs[cand].vec && !vec) ||
                          !config_ok(kConfigs[cand], ta, tb, vec, ilda, ildb, ldc, c_type)))
            continue;
        auto call = [&]() {
            return run(transa, transb, transc, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch,
                       ab_type, c_type, cand, stream, cand < 0 ? workspace : nullptr, cand < 0 ? workspace_bytes : 0,
                       false);
        };
        if (call() != TDG_SUCCESS) continue;                 // not servable (e.g. layout limits)
        if (hipEventRecord(e0, s) != hipSuccess) break;
        bool ok = true;
        for (int r = 0; r < reps && ok; ++r) ok = call() == TDG_SUCCESS;
        if (!ok || hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) break;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) break;
        if (best == -2 || ms < best_ms) {
            best = cand;
            best_ms = ms;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (best == -2) return fail(TDG_LAUNCH_FAILED, "no configuration could be timed: %s", g_err);
    {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        g_tune[TuneKey{dev, transa, transb, transc, ab_type, c_type, vec ? 1 : 0, M, N, K, batch}] = best;
    }
    if (best_config) *best_config = best;
    g_err[0] = '\0';
    return TDG_SUCCESS;
}

void tdg_autotune_clear(void) {
    std::lock_guard<std::mutex> lock(tdg::g_tune_mu);
    tdg::g_tune.clear();
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
    if (tdg::validate(0, transb, 0, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, batch > 1 ? (M - 1) * ldc + N : 0, batch,
                      ab_type, c_type, false) != TDG_SUCCESS)
        return -1;
    const bool vec = tdg::vec_ok(0, transb, M, N, K, A, lda, 0, B, ldb, 0, batch);
    int cus = 256, dev = -1;   // the MI355X count when no device is current
    if (tdg::check_device(&cus, &dev) != TDG_SUCCESS) cus = 256, dev = -1;
    tdg::g_err[0] = '\0';
    if (dev >= 0) {
        const int t = tdg::tuned_config(tdg::TuneKey{dev, 0, transb, 0, ab_type, c_type, vec ? 1 : 0, M, N, K, batch});
        if (t >= 0) return t;
    }
    return tdg::choose(0, transb, vec, M, N, K, batch, lda, ldb, ldc, c_type, cus);
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
