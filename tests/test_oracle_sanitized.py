"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, gcc) and driven through a small C program: every entry
point, including argument rejection and row subsets, must run clean."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
double orc_decode(int fmt, uint16_t bits);
uint16_t orc_encode(int fmt, double x);
int orc_gemm(int transb, int fmt, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda, int64_t sA,
             const uint16_t *B, int64_t ldb, int64_t sB, double *C, int64_t ldc, int64_t sC, int64_t batch,
             const int64_t *rows, int64_t nrows, int nthreads);
int orc_tiled_gemm(int transb, int fmt, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                   const uint16_t *B, int64_t ldb, int64_t BM, int64_t BN, int64_t BK, int acc_fmt, int out_fmt,
                   int drop_last_k, double *C, int64_t ldc);
int orc_tile_geometry(int64_t M, int64_t N, int64_t K, int64_t BM, int64_t BN, int64_t BK, int64_t i, int64_t j,
                      int64_t p, int64_t *g);
double orc_decode_f8(int fmt, uint8_t bits);
double orc_decode_e8m0(uint8_t bits);
int orc_gemm_f8(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda, int afmt, const uint8_t *B,
                int64_t ldb, int bfmt, const uint8_t *XA, int64_t ldxa, const uint8_t *XB, int64_t ldxb,
                int64_t block, const float *SA, int64_t inc_sa, const float *SB, int64_t inc_sb, double *C,
                int64_t ldc, int nthreads);
static int f8_cases(void) {
    const int64_t M = 13, N = 11, K = 70, nb = 3;
    uint8_t *A = malloc(M * K), *B = malloc(N * K), *XA = malloc(M * nb), *XB = malloc(N * nb);
    float *SA = malloc(sizeof(float) * M), *SB = malloc(sizeof(float) * N);
    double *C = malloc(sizeof(double) * M * N);
    for (int v = 0; v < 256; ++v) { orc_decode_f8(4, (uint8_t)v); orc_decode_f8(5, (uint8_t)v); orc_decode_e8m0((uint8_t)v); }
    for (int64_t i = 0; i < M * K; ++i) A[i] = (uint8_t)((i * 37) & 0x77);
    for (int64_t i = 0; i < N * K; ++i) B[i] = (uint8_t)((i * 11) & 0x7B);
    for (int64_t i = 0; i < M * nb; ++i) XA[i] = (uint8_t)(120 + i % 9);
    for (int64_t i = 0; i < N * nb; ++i) XB[i] = (uint8_t)(125 + i % 5);
    for (int64_t i = 0; i < M; ++i) SA[i] = 0.5f + (float)i / 16;
    for (int64_t i = 0; i < N; ++i) SB[i] = 1.5f - (float)i / 32;
    int bad = 0;
    bad |= orc_gemm_f8(M, N, K, A, K, 4, B, K, 5, XA, nb, XB, nb, 32, SA, 1, SB, 1, C, N, 3);
    bad |= orc_gemm_f8(M, N, K, A, K, 5, B, K, 4, NULL, 0, XB, nb, 32, SA, 0, NULL, 0, C, N, 1);
    bad |= orc_gemm_f8(M, N, 0, A, K, 4, B, K, 4, NULL, 0, NULL, 0, 32, NULL, 0, NULL, 0, C, N, 2);
    bad |= orc_gemm_f8(M, N, K, A, K, 4, B, K, 4, XA, nb - 1, NULL, 0, 32, NULL, 0, NULL, 0, C, N, 2) == 0;
    bad |= orc_gemm_f8(M, N, K, A, K, 3, B, K, 4, NULL, 0, NULL, 0, 32, NULL, 0, NULL, 0, C, N, 2) == 0;
    free(A); free(B); free(XA); free(XB); free(SA); free(SB); free(C);
    return bad;
}
int main(void) {
    if (f8_cases()) { printf("f8 cases failed\n"); return 9; }
    for (int f = 0; f < 2; ++f)
        for (int v = 0; v < 65536; ++v) {
            double d = orc_decode(f, (uint16_t)v);
            if (d == d && orc_encode(f, d) != (uint16_t)v && !(d == 0.0)) { printf("roundtrip %d %d\n", f, v); return 1; }
        }
    const int64_t M = 37, N = 29, K = 45, batch = 3;
    uint16_t *A = malloc(sizeof(uint16_t) * M * K * batch), *B = malloc(sizeof(uint16_t) * K * N * batch);
    double *C = malloc(sizeof(double) * M * N * batch), *T = malloc(sizeof(double) * M * N);
    for (int64_t i = 0; i < M * K * batch; ++i) A[i] = orc_encode(0, (double)((i * 7) % 5 - 2));
    for (int64_t i = 0; i < K * N * batch; ++i) B[i] = orc_encode(0, (double)((i * 3) % 5 - 2));
    for (int tb = 0; tb < 2; ++tb) {
        if (orc_gemm(tb, 0, M, N, K, A, K, M * K, B, tb ? K : N, K * N, C, N, M * N, batch, NULL, 0, 4)) return 2;
        int64_t rows[3] = {0, 17, 36};
        if (orc_gemm(tb, 1, M, N, K, A, K, M * K, B, tb ? K : N, K * N, C, N, 3 * N, batch, rows, 3, 2)) return 3;
        if (orc_tiled_gemm(tb, 0, M, N, K, A, K, B, tb ? K : N, 16, 8, 32, 2, 0, 0, T, N)) return 4;
        if (orc_tiled_gemm(tb, 0, M, N, K, A, K, B, tb ? K : N, 64, 64, 64, 1, 1, 1, T, N)) return 5;
    }
    if (orc_gemm(0, 0, -1, 2, 2, A, 2, 0, B, 2, 0, C, 2, 0, 1, NULL, 0, 1) == 0) return 6;
    int64_t g[27];
    if (orc_tile_geometry(65, 97, 130, 64, 64, 64, 1, 1, 2, g) || g[0] != 2 || g[1] != 2 || g[2] != 3) return 7;
    free(A); free(B); free(C); free(T);
    printf("ok\n");
    return 0;
}
"""


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "driver"
    cmd = [gcc, "-O1", "-g", "-std=c11", "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-ffp-contract=off", str(drv), os.path.join(ROOT, "oracle", "gemm_oracle.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
