/*
 * gemm_oracle.c -- CPU oracle for the tiled dense GEMM (TEST INFRASTRUCTURE).
 *
 * This file is the slow, obviously-correct reference that the GPU library is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or constant
 * with the HIP library: the number formats are decoded/encoded here from the
 * IEEE-754 definitions, and the product is the plain definition of a matrix
 * product summed in binary64.
 *
 * Sources (web pages; section names given in the pages' own headings):
 *   [NT]  studypath, "01.3.4 task3 appendix: NineToothed GEMM syntax primer"
 *         s1 nested tensor layers, s3 tracing one read (index map),
 *         s4 why M,N are outer and K is a loop, s5 tail tiles and masks,
 *         s6 what float32 accumulation keeps, s8 exercises.
 *   [CQ]  Croqtile tutorial ch.4 "tensor contraction: mma syntax", the
 *         four-step fill/load/multiply/store rhythm and the [N,K] rhs of
 *         its warp-level kernel (the "TN" form C = A * B^T).
 *
 * Functions:
 *   orc_decode        fp16 / bf16 bit pattern -> exact double.
 *   orc_encode        double -> fp16 / bf16 bits, IEEE round-to-nearest-even.
 *   orc_gemm          C[b,i,j] = sum_{p<K} A[b,i,p] * Bt[b,p,j], p ascending,
 *                     binary64, Bt = B (NN) or B^T (TN).  Whole rows or a
 *                     listed subset of rows; threads split rows only, so every
 *                     output is one sequential sum.
 *   orc_tiled_gemm    the [NT] tiled algorithm written out step by step: a
 *                     grid of (cdiv(M,BM), cdiv(N,BN)) programs, each zeroing
 *                     a BM x BN accumulator, looping p over cdiv(K,BK) K tiles,
 *                     reading masked tiles (out-of-range -> 0), adding the
 *                     tile product and storing under the output mask.  The
 *                     accumulator precision is a parameter (binary64,
 *                     binary32 or binary16) so the [NT] s6 example can be
 *                     reproduced; a flag drops the last K tile, a planted
 *                     mistake used only as a negative control by the tests.
 *   orc_tile_geometry grid sizes, K-step count and, for one (i, j, p), the
 *                     nominal and valid element ranges of the A tile, B tile
 *                     and output tile ([NT] s3, s4, s5).
 *   orc_decode_f8     E4M3 / E5M2 bit pattern -> exact double ([CQ] FP8
 *                     operands; bit layouts from the OCP 8-bit formats).
 *   orc_decode_e8m0   E8M0 block-scale byte -> 2^(e - 127).
 *   orc_gemm_f8       the scaled 8-bit TN product: per K block, the block's
 *                     contraction times the two operands' block scales,
 *                     summed over blocks, then times the row scales ([CQ]
 *                     per-tile scaled contraction and the separate scale
 *                     statement).
 *
 * Build: gcc -O3 -fPIC -shared -pthread -ffp-contract=off (see build.py).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element formats of the oracle.  Values are this file's own. */
enum { ORC_FMT_F16 = 0, ORC_FMT_BF16 = 1, ORC_FMT_F32 = 2, ORC_FMT_F64 = 3 };

/* Return codes. */
enum { ORC_OK = 0, ORC_BAD_ARG = -1, ORC_NO_MEM = -2 };

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits (the
 * upper half of a binary32).  Normal value (1 + f / 2^mb) * 2^(e - bias);
 * subnormal (e == 0) f * 2^(1 - bias - mb); e all-ones is inf (f == 0) or NaN. */
static void fmt_params(int fmt, int *ebits, int *mbits) {
    if (fmt == ORC_FMT_F16) { *ebits = 5; *mbits = 10; }
    else { *ebits = 8; *mbits = 7; }
}

double orc_decode(int fmt, uint16_t bits) {
    int eb, mb;
    fmt_params(fmt, &eb, &mb);
    const int bias = (1 << (eb - 1)) - 1;
    const int emax_field = (1 << eb) - 1;
    const int sign = (bits >> 15) & 1;
    const int e = (bits >> mb) & emax_field;
    const int f = bits & ((1 << mb) - 1);
    double v;
    if (e == 0) {
        v = ldexp((double)f, 1 - bias - mb);
    } else if (e == emax_field) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)((1 << mb) + f), e - bias - mb);
    }
    return sign ? -v : v;
}

/* Round a double to the nearest representable value of the format, ties to
 * even, overflow to +-inf; return the bit pattern.  The input is taken as the
 * exact value, so the result is a single correct rounding. */
uint16_t orc_encode(int fmt, double x) {
    int eb, mb;
    fmt_params(fmt, &eb, &mb);
    const int bias = (1 << (eb - 1)) - 1;
    const int emax_field = (1 << eb) - 1;
    const int emin = 1 - bias;                 /* exponent of the smallest normal */
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | (emax_field << mb) | (1 << (mb - 1)));
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | (emax_field << mb));
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);                              /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < emin) E = emin;                     /* subnormal range: fixed quantum */
    const double quantum = ldexp(1.0, E - mb);  /* spacing of values near a */
    const double n = nearbyint(a / quantum);    /* a/quantum is exact; RNE */
    const double v = n * quantum;
    /* largest finite value: (2 - 2^-mb) * 2^(emax_field - 1 - bias) */
    const double maxfin = ldexp((double)((2 << mb) - 1), emax_field - 1 - bias - mb);
    if (v > maxfin) return (uint16_t)(sign | (emax_field << mb));
    if (v < ldexp(1.0, emin)) {                 /* subnormal (or zero) */
        return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, emin - mb)));
    }
    frexp(v, &e2);
    E = e2 - 1;
    const int frac = (int)(v / ldexp(1.0, E - mb)) - (1 << mb);
    return (uint16_t)(sign | ((E + bias) << mb) | frac);
}

/* Bulk helpers for the Python side. */
void orc_decode_array(int fmt, const uint16_t *bits, double *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_decode(fmt, bits[i]);
}

void orc_encode_array(int fmt, const double *x, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_encode(fmt, x[i]);
}

/* ------------------------------------------------------------------------ */
/* Plain GEMM: the definition, summed in binary64                            */
/* ------------------------------------------------------------------------ */

/* Element p,j of the right operand as the product uses it: B[p,j] for NN
 * (B stored K x N, row stride ldb) and B[j,p] for TN (B stored N x K). */
static inline int64_t b_index(int transb, int64_t p, int64_t j, int64_t ldb) {
    return transb ? j * ldb + p : p * ldb + j;
}

typedef struct {
    int transb, fmt;
    int64_t N, K, lda, ldb, ldc;
    const double *Ad;          /* decoded A rows, K per row, for the rows below */
    const double *Bd;          /* decoded B, K x N (already as Bt[p][j]) */
    const int64_t *rows;       /* rows of this batch entry to compute */
    int64_t nrows;
    double *C;                 /* output, row r of the subset at C + r * ldc */
    int64_t r0, r1;            /* this thread's range within rows[] */
} gemm_job;

static void *gemm_worker(void *arg) {
    gemm_job *job = (gemm_job *)arg;
    const int64_t N = job->N, K = job->K;
    for (int64_t r = job->r0; r < job->r1; ++r) {
        const double *arow = job->Ad + r * K;
        double *crow = job->C + r * job->ldc;
        for (int64_t j = 0; j < N; ++j) crow[j] = 0.0;
        /* C[i, j] += A[i, p] * Bt[p, j] for p = 0, 1, ..., K-1 in order. */
        for (int64_t p = 0; p < K; ++p) {
            const double a = arow[p];
            const double *brow = job->Bd + p * N;
            for (int64_t j = 0; j < N; ++j) crow[j] += a * brow[j];
        }
    }
    return NULL;
}

/*
 * orc_gemm: for every batch entry b and every listed row i (all M rows if
 * rows == NULL), C[b][r][j] = sum_{p=0}^{K-1} dec(A[b,i,p]) * dec(Bt[b,p,j]),
 * where r is i's position in the list.  A is M x K row-major (lda), B is
 * K x N (transb == 0, NN) or N x K (transb == 1, TN) row-major (ldb), with
 * element strides sA/sB between batch entries; C is binary64 with row stride
 * ldc and batch stride sC.  K == 0 gives zeros (the empty sum).
 */
int orc_gemm(int transb, int fmt, int64_t M, int64_t N, int64_t K,
             const uint16_t *A, int64_t lda, int64_t sA,
             const uint16_t *B, int64_t ldb, int64_t sB,
             double *C, int64_t ldc, int64_t sC, int64_t batch,
             const int64_t *rows, int64_t nrows, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || batch < 0) return ORC_BAD_ARG;
    if (fmt != ORC_FMT_F16 && fmt != ORC_FMT_BF16) return ORC_BAD_ARG;
    if (lda < K || ldb < (transb ? K : N) || ldc < N) return ORC_BAD_ARG;
    if (rows == NULL) nrows = M;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return ORC_BAD_ARG;
    if (nthreads < 1) nthreads = 1;
    if (nrows == 0 || N == 0 || batch == 0) return ORC_OK;

    /* All 65536 bit patterns decoded once; element decoding is a lookup. */
    double *lut = (double *)malloc(sizeof(double) * 65536);
    if (!lut) return ORC_NO_MEM;
    for (int v = 0; v < 65536; ++v) lut[v] = orc_decode(fmt, (uint16_t)v);
    double *Ad = (double *)malloc(sizeof(double) * (size_t)(nrows * (K ? K : 1)));
    double *Bd = (double *)malloc(sizeof(double) * (size_t)((K ? K : 1) * N));
    int64_t *all = NULL;
    if (!Ad || !Bd) { free(lut); free(Ad); free(Bd); return ORC_NO_MEM; }
    if (rows == NULL) {
        all = (int64_t *)malloc(sizeof(int64_t) * (size_t)M);
        if (!all) { free(lut); free(Ad); free(Bd); return ORC_NO_MEM; }
        for (int64_t i = 0; i < M; ++i) all[i] = i;
        rows = all;
    }
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    gemm_job *jobs = (gemm_job *)malloc(sizeof(gemm_job) * (size_t)nthreads);
    if (!tid || !jobs) { free(lut); free(Ad); free(Bd); free(all); free(tid); free(jobs); return ORC_NO_MEM; }

    for (int64_t b = 0; b < batch; ++b) {
        const uint16_t *Ab = A + b * sA;
        const uint16_t *Bb = B + b * sB;
        for (int64_t r = 0; r < nrows; ++r)
            for (int64_t p = 0; p < K; ++p)
                Ad[r * K + p] = lut[Ab[rows[r] * lda + p]];
        for (int64_t p = 0; p < K; ++p)
            for (int64_t j = 0; j < N; ++j)
                Bd[p * N + j] = lut[Bb[b_index(transb, p, j, ldb)]];
        int nt = nthreads;
        if (nt > nrows) nt = (int)nrows;
        for (int t = 0; t < nt; ++t) {
            gemm_job *jb = &jobs[t];
            jb->transb = transb; jb->fmt = fmt;
            jb->N = N; jb->K = K; jb->lda = lda; jb->ldb = ldb; jb->ldc = ldc;
            jb->Ad = Ad; jb->Bd = Bd; jb->rows = rows; jb->nrows = nrows;
            jb->C = C + b * sC;
            jb->r0 = nrows * t / nt;
            jb->r1 = nrows * (t + 1) / nt;
        }
        int started = 0;
        for (int t = 1; t < nt; ++t) {
            if (pthread_create(&tid[t], NULL, gemm_worker, &jobs[t]) != 0) break;
            started = t;
        }
        gemm_worker(&jobs[0]);
        for (int t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
        for (int t = started + 1; t < nt; ++t) gemm_worker(&jobs[t]);  /* spawn failure: run inline */
    }
    free(lut); free(Ad); free(Bd); free(all); free(tid); free(jobs);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Tiled algorithm of [NT], step by step                                     */
/* ------------------------------------------------------------------------ */

static int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Round an accumulator value to the chosen accumulator precision. */
static double acc_round(int acc_fmt, double x) {
    switch (acc_fmt) {
    case ORC_FMT_F64: return x;
    case ORC_FMT_F32: return (double)(float)x;
    case ORC_FMT_F16: return orc_decode(ORC_FMT_F16, orc_encode(ORC_FMT_F16, x));
    case ORC_FMT_BF16: return orc_decode(ORC_FMT_BF16, orc_encode(ORC_FMT_BF16, x));
    default: return x;
    }
}

/*
 * orc_tile_geometry: for a BM x BN x BK tiling of an M x N x K product,
 * write grid_m = cdiv(M,BM), grid_n = cdiv(N,BN), ksteps = cdiv(K,BK) into
 * g[0..2]; then for program (i, j) at K step p, the half-open element ranges
 *   g[3..6]   A tile rows [i*BM, (i+1)*BM), cols [p*BK, (p+1)*BK)   (nominal)
 *   g[7..10]  B tile rows [p*BK, (p+1)*BK), cols [j*BN, (j+1)*BN)   (nominal, B as K x N)
 *   g[11..14] output tile rows [i*BM, (i+1)*BM), cols [j*BN, (j+1)*BN)
 *   g[15..26] the same three tiles clipped to the matrices (the valid parts
 *             that the read and write masks of [NT] s5 admit)
 */
int orc_tile_geometry(int64_t M, int64_t N, int64_t K, int64_t BM, int64_t BN, int64_t BK,
                      int64_t i, int64_t j, int64_t p, int64_t *g) {
    if (M < 0 || N < 0 || K < 0 || BM < 1 || BN < 1 || BK < 1) return ORC_BAD_ARG;
    g[0] = cdiv64(M, BM); g[1] = cdiv64(N, BN); g[2] = cdiv64(K, BK);
    const int64_t nom[12] = {
        i * BM, (i + 1) * BM, p * BK, (p + 1) * BK,
        p * BK, (p + 1) * BK, j * BN, (j + 1) * BN,
        i * BM, (i + 1) * BM, j * BN, (j + 1) * BN };
    const int64_t lim[12] = { M, M, K, K, K, K, N, N, M, M, N, N };
    for (int q = 0; q < 12; ++q) {
        g[3 + q] = nom[q];
        g[15 + q] = nom[q] < lim[q] ? nom[q] : lim[q];
    }
    return ORC_OK;
}

/*
 * orc_tiled_gemm: the tiled program of [NT] for an NN (transb == 0) or TN
 * (transb == 1) product.  For every program (i, j) of the output grid:
 *   acc[r][s] = 0                                   (BM x BN, acc_fmt precision)
 *   for p in 0 .. cdiv(K,BK)-1 (all but the last if drop_last_k):
 *     lhs[r][t] = A[i*BM+r, p*BK+t] if i*BM+r < M and p*BK+t < K else 0
 *     rhs[t][s] = Bt[p*BK+t, j*BN+s] if p*BK+t < K and j*BN+s < N else 0
 *     acc[r][s] += lhs[r][t] * rhs[t][s] for t = 0 .. BK-1, each add rounded
 *     to acc_fmt
 *   C[i*BM+r, j*BN+s] = out(acc[r][s]) where i*BM+r < M and j*BN+s < N
 * out() is exact binary64 (out_fmt F64), a binary32 rounding (F32), or the
 * fp16/bf16 encoding decoded back (F16/BF16).  C is binary64 with row stride
 * ldc; elements outside the store mask are never written.
 */
int orc_tiled_gemm(int transb, int fmt, int64_t M, int64_t N, int64_t K,
                   const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                   int64_t BM, int64_t BN, int64_t BK, int acc_fmt, int out_fmt,
                   int drop_last_k, double *C, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0 || BM < 1 || BN < 1 || BK < 1) return ORC_BAD_ARG;
    if (fmt != ORC_FMT_F16 && fmt != ORC_FMT_BF16) return ORC_BAD_ARG;
    if (lda < K || ldb < (transb ? K : N) || ldc < N) return ORC_BAD_ARG;
    const int64_t gm = cdiv64(M, BM), gn = cdiv64(N, BN), gk = cdiv64(K, BK);
    double *acc = (double *)malloc(sizeof(double) * (size_t)(BM * BN));
    double *lhs = (double *)malloc(sizeof(double) * (size_t)(BM * BK));
    double *rhs = (double *)malloc(sizeof(double) * (size_t)(BK * BN));
    if (!acc || !lhs || !rhs) { free(acc); free(lhs); free(rhs); return ORC_NO_MEM; }
    const int64_t psteps = (drop_last_k && gk > 0) ? gk - 1 : gk;
    for (int64_t i = 0; i < gm; ++i) {
        for (int64_t j = 0; j < gn; ++j) {
            for (int64_t q = 0; q < BM * BN; ++q) acc[q] = 0.0;
            for (int64_t p = 0; p < psteps; ++p) {
                for (int64_t r = 0; r < BM; ++r)
                    for (int64_t t = 0; t < BK; ++t) {
                        const int64_t row = i * BM + r, col = p * BK + t;
                        lhs[r * BK + t] = (row < M && col < K)
                            ? orc_decode(fmt, A[row * lda + col]) : 0.0;
                    }
                for (int64_t t = 0; t < BK; ++t)
                    for (int64_t s = 0; s < BN; ++s) {
                        const int64_t row = p * BK + t, col = j * BN + s;
                        rhs[t * BN + s] = (row < K && col < N)
                            ? orc_decode(fmt, B[b_index(transb, row, col, ldb)]) : 0.0;
                    }
                for (int64_t r = 0; r < BM; ++r)
                    for (int64_t s = 0; s < BN; ++s) {
                        double a = acc[r * BN + s];
                        for (int64_t t = 0; t < BK; ++t)
                            a = acc_round(acc_fmt, a + lhs[r * BK + t] * rhs[t * BN + s]);
                        acc[r * BN + s] = a;
                    }
            }
            for (int64_t r = 0; r < BM; ++r)
                for (int64_t s = 0; s < BN; ++s) {
                    const int64_t row = i * BM + r, col = j * BN + s;
                    if (row < M && col < N) {
                        double v = acc[r * BN + s];
                        if (out_fmt == ORC_FMT_F16 || out_fmt == ORC_FMT_BF16)
                            v = orc_decode(out_fmt, orc_encode(out_fmt, v));
                        else if (out_fmt == ORC_FMT_F32)
                            v = (double)(float)v;
                        C[row * ldc + col] = v;
                    }
                }
        }
    }
    free(acc); free(lhs); free(rhs);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 8-bit floating-point operands with scales                                 */
/* ------------------------------------------------------------------------ */

/* The Croqtile tutorial ch.4 (the variants after the four-step rhythm: FP8
 * operands with per-tile scaling) names the operand types f8_e4m3 and f8_e5m2
 * and gives the scaled contraction: the product of an operand pair is
 * multiplied by the two operands' scales after the contraction, with no
 * separate dequantisation pass.  The pages do not define the bit layouts;
 * they are taken here from the OCP 8-bit floating point formats:
 *   E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits.  No infinities: the
 *         all-ones exponent is an ordinary binade except for fraction 7,
 *         which is NaN, so the largest finite value is 1.75 * 2^8 = 448.
 *   E5M2: 1 sign, 5 exponent (bias 15), 2 fraction bits, binary16-like: the
 *         all-ones exponent is inf (fraction 0) or NaN.
 * Both have subnormals f * 2^(1 - bias - fraction_bits) at exponent 0.
 * The block scales are E8M0 (OCP microscaling): 8 exponent bits, no sign and
 * no fraction, value 2^(e - 127), 0xFF is NaN. */
enum { ORC_FMT_E4M3 = 4, ORC_FMT_E5M2 = 5 };

double orc_decode_f8(int fmt, uint8_t bits) {
    const int eb = (fmt == ORC_FMT_E4M3) ? 4 : 5;
    const int mb = 7 - eb;
    const int bias = (1 << (eb - 1)) - 1;
    const int emax_field = (1 << eb) - 1;
    const int sign = bits >> 7;
    const int e = (bits >> mb) & emax_field;
    const int f = bits & ((1 << mb) - 1);
    double v;
    if (fmt == ORC_FMT_E4M3 && e == emax_field && f == (1 << mb) - 1) {
        v = NAN;
    } else if (fmt == ORC_FMT_E5M2 && e == emax_field) {
        v = (f == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        v = ldexp((double)f, 1 - bias - mb);
    } else {
        v = ldexp((double)((1 << mb) + f), e - bias - mb);
    }
    return sign ? -v : v;
}

double orc_decode_e8m0(uint8_t bits) {
    return bits == 0xFF ? NAN : ldexp(1.0, (int)bits - 127);
}

void orc_decode_f8_array(int fmt, const uint8_t *bits, double *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_decode_f8(fmt, bits[i]);
}

void orc_decode_e8m0_array(const uint8_t *bits, double *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_decode_e8m0(bits[i]);
}

typedef struct {
    int64_t N, K, block, nblk;
    const double *Ad, *Bd;     /* decoded A (M x K) and B (N x K), K per row */
    const double *XA, *XB;     /* decoded block scales, nblk per row (or NULL) */
    const double *SA, *SB;     /* row scales (or NULL) */
    double *C;
    int64_t ldc, r0, r1;
} f8_job;

static void *f8_worker(void *arg) {
    const f8_job *jb = (const f8_job *)arg;
    const int64_t N = jb->N, K = jb->K, blk = jb->block, nb = jb->nblk;
    for (int64_t i = jb->r0; i < jb->r1; ++i) {
        const double *a = jb->Ad + i * K;
        for (int64_t j = 0; j < N; ++j) {
            const double *b = jb->Bd + j * K;
            double total = 0.0;
            for (int64_t t = 0; t < nb; ++t) {
                /* the contraction over one block of K ... */
                double part = 0.0;
                const int64_t k1 = (t + 1) * blk < K ? (t + 1) * blk : K;
                for (int64_t k = t * blk; k < k1; ++k) part += a[k] * b[k];
                /* ... then the two operands' scales for that block */
                if (jb->XA) part *= jb->XA[i * nb + t];
                if (jb->XB) part *= jb->XB[j * nb + t];
                total += part;
            }
            if (jb->SA) total *= jb->SA[i];
            if (jb->SB) total *= jb->SB[j];
            jb->C[i * jb->ldc + j] = total;
        }
    }
    return NULL;
}

/*
 * orc_gemm_f8: C[i][j] = sa(i) * sb(j) * sum_t xa(i,t) * xb(j,t) *
 *                        sum_{k in block t} dec(A[i,k]) * dec(B[j,k])
 * in binary64, for A M x K (row stride lda, format afmt) and B N x K (row
 * stride ldb, format bfmt): the TN form C = A * B^T.  Block t covers
 * k = t*block .. min((t+1)*block, K) - 1.
 *   xa(i,t) = 2^(XA[i*ldxa + t] - 127) (E8M0), or 1 when XA is NULL; xb alike
 *             with XB, ldxb.
 *   sa(i)   = SA[i*inc_sa] (inc_sa 0: one scale for the whole operand), or 1
 *             when SA is NULL; sb alike.
 * K == 0 gives zeros.  Threads split the rows of C.
 */
int orc_gemm_f8(int64_t M, int64_t N, int64_t K,
                const uint8_t *A, int64_t lda, int afmt,
                const uint8_t *B, int64_t ldb, int bfmt,
                const uint8_t *XA, int64_t ldxa, const uint8_t *XB, int64_t ldxb, int64_t block,
                const float *SA, int64_t inc_sa, const float *SB, int64_t inc_sb,
                double *C, int64_t ldc, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || block < 1) return ORC_BAD_ARG;
    if ((afmt != ORC_FMT_E4M3 && afmt != ORC_FMT_E5M2) || (bfmt != ORC_FMT_E4M3 && bfmt != ORC_FMT_E5M2))
        return ORC_BAD_ARG;
    const int64_t nb = cdiv64(K, block);
    if (lda < K || ldb < K || ldc < N || (XA && ldxa < nb) || (XB && ldxb < nb) || inc_sa < 0 || inc_sb < 0)
        return ORC_BAD_ARG;
    if (nthreads < 1) nthreads = 1;
    if (M == 0 || N == 0) return ORC_OK;
    double lut_a[256], lut_b[256];
    for (int v = 0; v < 256; ++v) {
        lut_a[v] = orc_decode_f8(afmt, (uint8_t)v);
        lut_b[v] = orc_decode_f8(bfmt, (uint8_t)v);
    }
    const size_t kk = (size_t)(K ? K : 1), bb = (size_t)(nb ? nb : 1);
    double *Ad = (double *)malloc(sizeof(double) * (size_t)M * kk);
    double *Bd = (double *)malloc(sizeof(double) * (size_t)N * kk);
    double *xa = XA ? (double *)malloc(sizeof(double) * (size_t)M * bb) : NULL;
    double *xb = XB ? (double *)malloc(sizeof(double) * (size_t)N * bb) : NULL;
    double *sa = SA ? (double *)malloc(sizeof(double) * (size_t)M) : NULL;
    double *sb = SB ? (double *)malloc(sizeof(double) * (size_t)N) : NULL;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    f8_job *jobs = (f8_job *)malloc(sizeof(f8_job) * (size_t)nthreads);
    if (!Ad || !Bd || (XA && !xa) || (XB && !xb) || (SA && !sa) || (SB && !sb) || !tid || !jobs) {
        free(Ad); free(Bd); free(xa); free(xb); free(sa); free(sb); free(tid); free(jobs);
        return ORC_NO_MEM;
    }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) Ad[i * K + k] = lut_a[A[i * lda + k]];
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k) Bd[j * K + k] = lut_b[B[j * ldb + k]];
    for (int64_t i = 0; xa && i < M; ++i)
        for (int64_t t = 0; t < nb; ++t) xa[i * nb + t] = orc_decode_e8m0(XA[i * ldxa + t]);
    for (int64_t j = 0; xb && j < N; ++j)
        for (int64_t t = 0; t < nb; ++t) xb[j * nb + t] = orc_decode_e8m0(XB[j * ldxb + t]);
    for (int64_t i = 0; sa && i < M; ++i) sa[i] = (double)SA[i * inc_sa];
    for (int64_t j = 0; sb && j < N; ++j) sb[j] = (double)SB[j * inc_sb];
    int nt = nthreads;
    if (nt > M) nt = (int)M;
    for (int t = 0; t < nt; ++t) {
        f8_job *jb = &jobs[t];
        jb->N = N; jb->K = K; jb->block = block; jb->nblk = nb;
        jb->Ad = Ad; jb->Bd = Bd; jb->XA = xa; jb->XB = xb; jb->SA = sa; jb->SB = sb;
        jb->C = C; jb->ldc = ldc;
        jb->r0 = M * t / nt;
        jb->r1 = M * (t + 1) / nt;
    }
    int started = 0;
    for (int t = 1; t < nt; ++t) {
        if (pthread_create(&tid[t], NULL, f8_worker, &jobs[t]) != 0) break;
        started = t;
    }
    f8_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
    for (int t = started + 1; t < nt; ++t) f8_worker(&jobs[t]);
    free(Ad); free(Bd); free(xa); free(xb); free(sa); free(sb); free(tid); free(jobs);
    return ORC_OK;
}
