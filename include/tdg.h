/*
 * tdg.h -- tiled dense GEMM for AMD Instinct MI355X (gfx950): C ABI.
 *
 * Operation.  C = A * B ("NN", B stored K x N) or C = A * B^T ("TN", B stored
 * N x K), with fp16 or bf16 inputs, fp32 accumulation and fp16, bf16 or fp32
 * output.  Every output element is the full sum over K of products of input
 * elements:  C[i,j] = sum_{p<K} A[i,p] * Bt[p,j].
 *   - The product, its tile decomposition, the zero-filled reads past the
 *     matrix edges and the store mask of edge tiles follow the NineToothed
 *     GEMM primer (studypath task3 appendix), sections 3 (index map),
 *     4 (M and N over the grid, K as a loop inside one program) and
 *     5 (tail tiles: masked reads return 0, masked store).
 *   - The TN form is the [N, K] right operand of the warp-level kernel in the
 *     Croqtile tutorial, chapter 4 ("tensor contraction: mma syntax"),
 *     read as out[m,n] = sum_k lhs[m,k] * rhs[n,k].
 *   - fp32 accumulation follows section 6 of the NineToothed primer; the
 *     fp32 -> fp16/bf16 output conversion rounds to nearest even, overflow
 *     to +-inf.
 *
 * Layout.  All matrices are row-major.  Leading dimensions are row strides
 * in ELEMENTS: lda >= K; ldb >= N (NN) or ldb >= K (TN); ldc >= N.  Batched
 * calls add element strides between consecutive problems (strideA/B/C); the
 * problems are independent.  Every pointer must be aligned to its element
 * size (2 bytes for A, B and a 16-bit C, 4 bytes for an fp32 C); any leading
 * dimension is accepted.  16-byte aligned bases with leading dimensions and
 * contiguous extents that are multiples of 8 elements take the vectorised
 * path, the rest a slower predicated path with identical results.
 *
 * Ownership.  The caller allocates A, B and C in device memory (HBM) and
 * keeps them alive until the stream work completes.  The library allocates
 * no device memory, keeps no per-call state and never synchronises: each
 * call only validates its arguments and enqueues its kernels on `stream`
 * (a hipStream_t; NULL is the null stream) -- one launch, or two launches
 * over disjoint parts of C for a single problem whose 256 x 256 output
 * tiles leave a partial last round on the device's compute units (a band of
 * whole rounds of 256 x 256 tiles, then the rest in 128 x 128 tiles).  C is
 * fully overwritten (alpha = 1, beta = 0) and must not overlap A or B.
 *
 * Errors.  Argument errors are reported synchronously, before anything is
 * enqueued, through the return value; tdg_last_error() then describes the
 * cause (thread-local).  Faults inside a kernel surface at the caller's next
 * synchronisation, as for any HIP kernel.
 *   TDG_INVALID_VALUE  negative M, N, K or batch; M, N or K of 2^31 or more;
 *                      a NULL pointer with work to do; A, B or C not aligned
 *                      to its element size; a leading dimension too small, a
 *                      negative batch stride, or a strideC that lets the C
 *                      matrices of a batch overlap; an unknown dtype or a
 *                      dtype combination not offered; more than 2^31 - 1
 *                      output tiles of 64 x 64.
 *   TDG_NOT_SUPPORTED  the current device is not gfx950.
 *   TDG_LAUNCH_FAILED  the kernel launch was rejected by the HIP runtime.
 * Degenerate sizes: M == 0, N == 0 or batch == 0 do nothing and succeed;
 * K == 0 writes zeros to C (the empty sum).
 */
#ifndef TDG_H
#define TDG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TDG_ABI_VERSION 4

/* TDG_E4M3 and TDG_E5M2 are the 8-bit operand types of tdg_gemm_f8 only. */
typedef enum { TDG_F16 = 0, TDG_BF16 = 1, TDG_F32 = 2, TDG_E4M3 = 3, TDG_E5M2 = 4 } tdg_dtype;

typedef enum {
    TDG_SUCCESS = 0,
    TDG_INVALID_VALUE = 1,
    TDG_NOT_SUPPORTED = 2,
    TDG_LAUNCH_FAILED = 3
} tdg_status;

/* C (M x N) = A (M x K) * B (K x N).  ab_type in {TDG_F16, TDG_BF16} for both
 * inputs; c_type in {TDG_F16, TDG_BF16, TDG_F32}. */
tdg_status tdg_gemm_nn(int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda,
                       const void *B, int64_t ldb,
                       void *C, int64_t ldc,
                       tdg_dtype ab_type, tdg_dtype c_type, void *stream);

/* C (M x N) = A (M x K) * B^T with B stored N x K (row stride ldb >= K). */
tdg_status tdg_gemm_tn(int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda,
                       const void *B, int64_t ldb,
                       void *C, int64_t ldc,
                       tdg_dtype ab_type, tdg_dtype c_type, void *stream);

/* `batch` independent NN products; problem z uses A + z*strideA,
 * B + z*strideB, C + z*strideC (element offsets).  Each stride must be
 * nonnegative, and strideC must keep the C matrices disjoint
 * (strideC >= (M-1)*ldc + N when batch > 1). */
tdg_status tdg_gemm_nn_batched(int64_t M, int64_t N, int64_t K,
                               const void *A, int64_t lda, int64_t strideA,
                               const void *B, int64_t ldb, int64_t strideB,
                               void *C, int64_t ldc, int64_t strideC,
                               int64_t batch,
                               tdg_dtype ab_type, tdg_dtype c_type, void *stream);

/* `batch` independent TN products (B_z stored N x K). */
tdg_status tdg_gemm_tn_batched(int64_t M, int64_t N, int64_t K,
                               const void *A, int64_t lda, int64_t strideA,
                               const void *B, int64_t ldb, int64_t strideB,
                               void *C, int64_t ldc, int64_t strideC,
                               int64_t batch,
                               tdg_dtype ab_type, tdg_dtype c_type, void *stream);

/* Same as the batched calls, with the tile configuration forced: `config`
 * is an index in [0, tdg_num_configs()) or -1 for the library's own choice.
 * `transb` is 0 for NN and 1 for TN.  A forced configuration that cannot
 * serve the arguments (the vectorised path on misaligned operands) returns
 * TDG_INVALID_VALUE.  Meant for tests and tuning sweeps. */
tdg_status tdg_gemm_ex(int transb, int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda, int64_t strideA,
                       const void *B, int64_t ldb, int64_t strideB,
                       void *C, int64_t ldc, int64_t strideC,
                       int64_t batch,
                       tdg_dtype ab_type, tdg_dtype c_type, int config, void *stream);

/* Split-K calls.  The NineToothed primer (s4) keeps K as a loop inside one
 * program and names the alternative, splitting K over programs, together
 * with its cost: a merge step.  tdg_gemm_ws is tdg_gemm_ex with the
 * library's own choice of configuration plus a caller-owned workspace that
 * enables split-K schedules, in which some output tiles are each cut into K
 * slices run by separate workgroups; each slice writes an fp32 partial tile
 * into the workspace and the last slice to finish adds them in slice order
 * and writes C:
 *   - few tiles with a long K (fewer 128 x 128 tiles than compute units):
 *     every tile is cut into slices;
 *   - a single problem whose 256 x 256 tiles leave a partial last round
 *     (e.g. 289 tiles on 256 CUs): one launch in which the tiles of whole
 *     rounds are whole work items and the tiles of the partial round are
 *     cut into slices, when no band of whole rounds can be cut off or the
 *     rest of such a cut would fill fewer than half of the compute units
 *     (otherwise the band and the rest run as two launches, without a
 *     workspace).
 * The result is the same sum with another rounding order (bitwise equal for
 * exactly representable sums), and it is deterministic: the same call on the
 * same device gives the same bits.
 *
 * workspace: device memory, 256-byte aligned, at least
 *   tdg_gemm_workspace_size(...) bytes for these sizes, zero-filled before its
 *   first use and not written by the caller afterwards (each call leaves
 *   behind what the next call needs: its counters back at zero).  NULL
 *   (with workspace_bytes 0) runs without split-K.  Calls that may overlap in
 *   time (other streams, other threads) must not share a workspace.
 * Errors: as tdg_gemm_ex, plus TDG_INVALID_VALUE for a misaligned or too
 * small workspace.
 * The library still allocates nothing; the caller owns the workspace. */
tdg_status tdg_gemm_ws(int transb, int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda, int64_t strideA,
                       const void *B, int64_t ldb, int64_t strideB,
                       void *C, int64_t ldc, int64_t strideC,
                       int64_t batch,
                       tdg_dtype ab_type, tdg_dtype c_type,
                       void *workspace, size_t workspace_bytes, void *stream);

/* The general call: any storage order of A, B and C.  The Croqtile
 * tutorial, chapter 4, gives the contraction layout variants (row.row,
 * row.col: which operands are stored K-contiguous) and a transposed store of
 * the accumulator tile (mma.store.transp, for a consumer that wants the other
 * major order); this call offers all of them:
 *   transa 0: A stored M x K (lda >= K);  1: A stored K x M (lda >= M).
 *   transb 0: B stored K x N (ldb >= N);  1: B stored N x K (ldb >= K).
 *   transc 0: C stored M x N (ldc >= N);  1: C stored N x M (ldc >= M), i.e.
 *             element (i, j) of the product at C[j * ldc + i].
 * C[i,j] = sum_{p<K} A(i,p) * B(p,j) as everywhere else; strides, dtypes,
 * workspace and errors as tdg_gemm_ws (strideC must keep the stored C
 * matrices disjoint).  A transposed store is the exchanged product
 * C^T = B^T A^T, run by the same kernels.  Layouts that need an A stored
 * K x M (transa 1 with transc 0, or transb 0 with transc 1) run on the
 * vectorised kernel only: 16-byte aligned A and B, leading dimensions, batch
 * strides and contiguous extents multiples of 8 elements; other operands
 * return TDG_NOT_SUPPORTED. */
tdg_status tdg_gemm(int transa, int transb, int transc, int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t lda, int64_t strideA,
                    const void *B, int64_t ldb, int64_t strideB,
                    void *C, int64_t ldc, int64_t strideC,
                    int64_t batch,
                    tdg_dtype ab_type, tdg_dtype c_type,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes tdg_gemm_ws needs for these sizes on a device with
 * `num_cus` compute units (0: the current device); 0 when no split-K
 * schedule would be used.  An upper bound: operands that cannot take the
 * vectorised kernels need none.  Also valid for tdg_gemm with any
 * transa, transb, transc (the tile counts do not depend on them). */
size_t tdg_gemm_workspace_size(int transb, int64_t M, int64_t N, int64_t K, int64_t batch, int num_cus);

/* An upper bound of tdg_gemm_workspace_size over every problem, on a device
 * with `num_cus` compute units (0: the current device; 0 is returned when
 * no gfx950 device is current): a workspace of this size serves any call,
 * so a caller can allocate one per stream once and never replace it (for
 * instance when calls are captured in a HIP graph, whose replays keep
 * using the pointer they were captured with).  A graph replay and an eager
 * call that share a workspace must not overlap in time. */
size_t tdg_gemm_workspace_bound(int num_cus);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops and harnesses that forbid allocation.  The same
 * product as tdg_gemm (same arguments, storage orders, checks and results,
 * bit for bit), with the split-K workspace taken from a scratch array that is
 * part of the library's device code: TDG_NOALLOC_SCRATCH_BYTES on every GPU
 * the library runs on, held from the library's load until the process ends.
 * The call allocates nothing and frees nothing.
 *   - Every call on one GPU uses that GPU's array, which keeps what the last
 *     call left (its arrival counters back at zero).  Calls that may overlap
 *     in time on one GPU -- on several streams, from several threads, or a
 *     graph replay beside an eager call -- race on the array and must not be
 *     issued; serialise them (one stream) or use tdg_gemm with a workspace
 *     per stream.
 *   - TDG_INVALID_VALUE when the device's split-K schedule could need more
 *     than TDG_NOALLOC_SCRATCH_BYTES (a device with more than 256 compute
 *     units), besides tdg_gemm's own errors. */
#define TDG_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u + 4096u)
tdg_status tdg_gemm_noalloc(int transa, int transb, int transc, int64_t M, int64_t N, int64_t K,
                            const void *A, int64_t lda, int64_t strideA,
                            const void *B, int64_t ldb, int64_t strideB,
                            void *C, int64_t ldc, int64_t strideC,
                            int64_t batch,
                            tdg_dtype ab_type, tdg_dtype c_type, void *stream);

/* Autotuning (tile selection by measurement).  Times every tile
 * configuration that can serve these arguments, and the library's own
 * schedule, `reps` calls each on the caller's buffers and stream, and records
 * the fastest for this process: later automatic calls (tdg_gemm*,
 * tdg_gemm_nn/tn*) on the same device with the same storage orders, sizes,
 * types, batch and alignment class run that configuration, and
 * tdg_select_config reports it.  Unlike every other call this one
 * synchronises `stream` (it waits for its timing events) and writes C
 * (with the product, many times).  *best_config receives the configuration
 * index, or -1 when the library's own schedule won.  reps in [1, 1000].
 * Errors as tdg_gemm, plus TDG_LAUNCH_FAILED when nothing could be timed. */
tdg_status tdg_autotune(int transa, int transb, int transc, int64_t M, int64_t N, int64_t K,
                        const void *A, int64_t lda, int64_t strideA,
                        const void *B, int64_t ldb, int64_t strideB,
                        void *C, int64_t ldc, int64_t strideC,
                        int64_t batch,
                        tdg_dtype ab_type, tdg_dtype c_type,
                        void *workspace, size_t workspace_bytes,
                        int reps, int *best_config, void *stream);

/* Forget every autotuning result of this process. */
void tdg_autotune_clear(void);

/* Number of tile configurations and the name of configuration `config`
 * (e.g. "256x256x64_w2x2_vec"); NULL for an index out of range. */
int tdg_num_configs(void);
const char *tdg_config_name(int config);

/* The configuration the library would choose for these arguments (pointers
 * are inspected for alignment only, never dereferenced); -1 on bad args.
 * A problem tuned by tdg_autotune (transa = transc = 0) reports the tuned
 * configuration. */
int tdg_select_config(int transb, int64_t M, int64_t N, int64_t K,
                      const void *A, int64_t lda, const void *B, int64_t ldb,
                      const void *C, int64_t ldc, int64_t batch,
                      tdg_dtype ab_type, tdg_dtype c_type);

/* 8-bit floating-point operands with scales.  The Croqtile tutorial,
 * chapter 4 (the variants after the four-step rhythm: quantised operands
 * with per-tile scaling), has FP8 operands (f8_e4m3, f8_e5m2) whose scales
 * multiply the contraction after it is formed, in the same kernel -- fused
 * into the contraction, or as a separate statement on the accumulator.  The
 * bit layouts are the OCP 8-bit formats: E4M3 (bias 7, no infinities,
 * S.1111.111 is NaN, largest finite 448) and E5M2 (bias 15, IEEE-like
 * infinities and NaNs); both with subnormals.
 *
 * C (M x N) = A * B^T with A stored M x K and B stored N x K (row-major, row
 * strides lda, ldb >= K, in bytes = elements), fp32 accumulation:
 *   C[i,j] = sa(i) * sb(j) * sum_t xa(i,t) * xb(j,t) * sum_{k in block t} A[i,k] * B[j,k]
 * where block t is k = 32t .. min(32t+32, K) - 1 and
 *   xa(i,t) = 2^(block_scale_a[i * ld_bsa + t] - 127)   E8M0 bytes, 1 if NULL
 *   xb(j,t) = 2^(block_scale_b[j * ld_bsb + t] - 127)   (likewise)
 *   sa(i)   = scale_a[i * inc_a]   fp32; inc_a 0 = one scale for A; 1 if NULL
 *   sb(j)   = scale_b[j * inc_b]   (likewise for the rows of B)
 * The block scales are the scale operands of the MFMA itself (the fused
 * form, 32-element blocks as the gfx950 instruction takes them); the row
 * scales multiply the fp32 sums in the epilogue (the separate statement),
 * before the conversion to c_type (round to nearest even).  The E8M0 byte
 * 0xFF (NaN) is not a valid scale.
 *
 * a_type, b_type: TDG_E4M3 or TDG_E5M2, independently.  c_type: TDG_F16,
 * TDG_BF16 or TDG_F32.  transc 1 stores C transposed: N x M, ldc >= M,
 * element (i, j) at C[j * ldc + i] (the product with the operands and their
 * scales exchanged).  config: -1 for the library's choice, or an index in
 * [0, tdg_f8_num_configs()).
 * Requirements, else TDG_NOT_SUPPORTED: A and B 16-byte aligned, lda, ldb
 * and K multiples of 16; block-scale arrays 16-byte aligned with ld_bsa,
 * ld_bsb multiples of 16 (and >= ceil(K/32), else TDG_INVALID_VALUE), each
 * an M x ld_bsa (N x ld_bsb) byte array of which only the first ceil(K/32)
 * bytes of a row are used.  Row scales 4-byte aligned.
 * Ownership, errors and degenerate sizes as for the other calls (K == 0
 * writes zeros; M == 0 or N == 0 does nothing). */
tdg_status tdg_gemm_f8(int transc, int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda, tdg_dtype a_type,
                       const void *B, int64_t ldb, tdg_dtype b_type,
                       const void *block_scale_a, int64_t ld_bsa,
                       const void *block_scale_b, int64_t ld_bsb,
                       const float *scale_a, int64_t inc_a,
                       const float *scale_b, int64_t inc_b,
                       void *C, int64_t ldc, tdg_dtype c_type, int config, void *stream);

/* Number of 8-bit tile configurations and the name of one (NULL out of range). */
int tdg_f8_num_configs(void);
const char *tdg_f8_config_name(int config);

const char *tdg_status_string(tdg_status status);
/* Human-readable cause of this thread's most recent non-success ("" if none). */
const char *tdg_last_error(void);
int tdg_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TDG_H */
