/*
 * c_abi_check.c -- drives liblsec.so from plain C (no Python, no PyTorch):
 * device buffers from hipMalloc, inputs from the seeded generator
 * (synth/libsynth.so), expected values from the CPU oracle
 * (oracle/liblsec_oracle.so), comparisons with the tolerances of the GPU
 * parity tests. TEST INFRASTRUCTURE: built by __graft_entry__.build(), run by
 * tests/test_gpu_zz_c_abi.py.
 *
 * Cases: the combine (bf16, tiled path, base e, global LSE), the combine
 * (fp16, row path, base 2), an fp32 result from bf16 partials, pack_send
 * (bit-exact; also over more tiles than the pack's grid has blocks),
 * unpack_combine on the oracle's packed buffer, unpack (bit-exact), the
 * token-major merge (both token dims), the corrected partial, the combine of
 * strided receive planes (with and without the valid count on the device), the
 * path diagnostics, the status strings and the error statuses of invalid
 * arguments (nothing is launched).
 * Exit status 0 when every case passes, 1 on a mismatch, 2 when no GPU is
 * usable.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lsec.h"

/* synth/libsynth.so */
uint64_t synth_key(uint64_t seed, uint32_t cfg, uint32_t tensor, uint32_t sub);
int synth_fill(uint64_t key, int64_t off, int64_t n, int dist, double a, double b, int out,
               void* dst, int nthreads);
int synth_u01(uint64_t key, int64_t off, int64_t n, double* dst, int nthreads);

/* oracle/liblsec_oracle.so */
int oracle_bits_to_f64(const void* bits, int dtype, int64_t n, double* out);
int oracle_lse_combine(const void* outputs, int dtype, const float* lses, int64_t N, int64_t B,
                       int64_t H, int64_t D, int base2, double* y, double* L);
int oracle_pack_send(const void* out, const float* lse, int64_t N, int64_t B, int64_t H,
                     int64_t D, int64_t E, void* send);
int oracle_unpack(const void* recv, int64_t N, int64_t B, int64_t Hl, int64_t D, int64_t E,
                  void* outputs, float* lses);
int oracle_unpack_combine(const void* recv, int dtype, int64_t N, int64_t B, int64_t Hl,
                          int64_t D, int base2, double* y, double* L);
int oracle_merge(const void* outputs, int dtype, const float* lses, int64_t N, int64_t A,
                 int64_t C, int64_t D, int token_dim, int base2, double* y, double* L);
int oracle_correct_partial(const float* lses, int64_t N, int64_t rank, const void* partial,
                           int dtype, int64_t B, int64_t H, int64_t D, int base2, double* y,
                           double* L);

enum { DIST_UNIFORM = 0, DIST_NORMAL = 1 };
enum { OUT_F32 = 1, OUT_BF16 = 2, OUT_F16 = 3 };

static int failures = 0;

#define HIP_OK(x)                                                                   \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(1);                                                                \
        }                                                                           \
    } while (0)

static void check(int ok, const char* what) {
    printf("%-58s %s\n", what, ok ? "ok" : "FAILED");
    fflush(stdout);
    if (!ok) ++failures;
}

static void* dev_copy(const void* host, size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
    if (bytes) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

/* Partial outputs [N,B,H,D] (16-bit patterns) and LSEs [N,B,H] with a share
 * of NaN / +inf / -inf entries drawn from a separate uniform stream. */
static void draw(uint32_t cfg, int out_kind, int64_t n_out, int64_t n_lse, uint16_t* o, float* l,
                 double lo, double hi) {
    synth_fill(synth_key(0, cfg, 1, 0), 0, n_out, DIST_NORMAL, 0.0, 1.0, out_kind, o, 1);
    synth_fill(synth_key(0, cfg, 2, 0), 0, n_lse, DIST_UNIFORM, lo, hi, OUT_F32, l, 1);
    double* u = malloc(sizeof(double) * (size_t)n_lse);
    synth_u01(synth_key(0, cfg, 3, 0), 0, n_lse, u, 1);
    for (int64_t i = 0; i < n_lse; ++i) {
        if (u[i] < 0.03) l[i] = NAN;
        else if (u[i] < 0.06) l[i] = INFINITY;
        else if (u[i] < 0.09) l[i] = -INFINITY;
    }
    free(u);
}

static double max_abs(const void* bits, int dtype, int64_t n) {
    double* v = malloc(sizeof(double) * (size_t)n);
    oracle_bits_to_f64(bits, dtype, n, v);
    double m = 0.0;
    for (int64_t i = 0; i < n; ++i)
        if (isfinite(v[i]) && fabs(v[i]) > m) m = fabs(v[i]);
    free(v);
    return m;
}

/* |y - y_ref| <= tol * M + 1e-6 (NaN where the oracle has NaN); LSE within 1e-5,
 * non-finite LSEs equal. y holds `rows * D` results of `res_dtype`. */
static int close_enough(const void* y, int res_dtype, const double* y_ref, int64_t n, double M,
                        const float* L, const double* L_ref, int64_t rows) {
    const double tol = res_dtype == LSEC_BF16 ? 8e-3 : (res_dtype == LSEC_FP16 ? 1e-3 : 2e-5);
    double* yv = malloc(sizeof(double) * (size_t)n);
    oracle_bits_to_f64(y, res_dtype == LSEC_FP32 ? 2 : res_dtype, n, yv);
    int ok = 1;
    for (int64_t i = 0; i < n && ok; ++i) {
        if (isnan(y_ref[i])) ok = isnan(yv[i]);
        else ok = fabs(yv[i] - y_ref[i]) <= tol * M + 1e-6;
    }
    free(yv);
    for (int64_t r = 0; L && r < rows && ok; ++r) {
        if (isfinite(L_ref[r])) ok = isfinite(L[r]) && fabs((double)L[r] - L_ref[r]) <= 1e-5;
        else ok = (double)L[r] == L_ref[r];
    }
    return ok;
}

static void combine_case(const char* name, uint32_t cfg, int64_t N, int64_t B, int64_t H,
                         int64_t D, int dtype, int base, int out_f32) {
    const int64_t rows = B * H, n_out = N * rows * D;
    uint16_t* o = malloc(sizeof(uint16_t) * (size_t)n_out);
    float* l = malloc(sizeof(float) * (size_t)(N * rows));
    draw(cfg, dtype == LSEC_BF16 ? OUT_BF16 : OUT_F16, n_out, N * rows, o, l, -5.0, 15.0);
    const size_t res_bytes = (size_t)(rows * D) * (out_f32 ? 4 : 2);
    void* d_o = dev_copy(o, sizeof(uint16_t) * (size_t)n_out);
    void* d_l = dev_copy(l, sizeof(float) * (size_t)(N * rows));
    void* d_y = NULL;
    float* d_L = NULL;
    HIP_OK(hipMalloc(&d_y, res_bytes));
    HIP_OK(hipMalloc((void**)&d_L, sizeof(float) * (size_t)rows));
    const int st = lsec_combine(d_o, (const float*)d_l, N, B, H, D,
                                dtype | (out_f32 ? LSEC_OUT_FP32 : 0), base, d_y, d_L, NULL);
    HIP_OK(hipDeviceSynchronize());
    void* y = malloc(res_bytes);
    float* L = malloc(sizeof(float) * (size_t)rows);
    HIP_OK(hipMemcpy(y, d_y, res_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(L, d_L, sizeof(float) * (size_t)rows, hipMemcpyDeviceToHost));
    double* y_ref = malloc(sizeof(double) * (size_t)(rows * D));
    double* L_ref = malloc(sizeof(double) * (size_t)rows);
    oracle_lse_combine(o, dtype, l, N, B, H, D, base == LSEC_BASE_2, y_ref, L_ref);
    check(st == LSEC_OK && close_enough(y, out_f32 ? LSEC_FP32 : dtype, y_ref, rows * D,
                                        max_abs(o, dtype, n_out), L, L_ref, rows),
          name);
    HIP_OK(hipFree(d_o));
    HIP_OK(hipFree(d_l));
    HIP_OK(hipFree(d_y));
    HIP_OK(hipFree(d_L));
    free(o), free(l), free(y), free(L), free(y_ref), free(L_ref);
}

static void packed_case(void) {
    const int64_t N = 4, B = 9, H = 8, D = 128, Hl = H / N, rows = B * H;
    const int64_t W = D + lsec_pack_dim(LSEC_BF16);
    uint16_t* o = malloc(sizeof(uint16_t) * (size_t)(rows * D));
    float* l = malloc(sizeof(float) * (size_t)rows);
    draw(40, OUT_BF16, rows * D, rows, o, l, -5.0, 15.0);
    l[0] = NAN;  /* a NaN payload must move as bits */
    const size_t send_bytes = sizeof(uint16_t) * (size_t)(N * B * Hl * W);
    void* d_o = dev_copy(o, sizeof(uint16_t) * (size_t)(rows * D));
    void* d_l = dev_copy(l, sizeof(float) * (size_t)rows);
    void* d_s = NULL;
    HIP_OK(hipMalloc(&d_s, send_bytes));
    int st = lsec_pack_send(d_o, (const float*)d_l, N, B, H, D, LSEC_BF16, d_s, NULL);
    HIP_OK(hipDeviceSynchronize());
    uint16_t* s = malloc(send_bytes);
    uint16_t* s_ref = malloc(send_bytes);
    HIP_OK(hipMemcpy(s, d_s, send_bytes, hipMemcpyDeviceToHost));
    oracle_pack_send(o, l, N, B, H, D, 2, s_ref);
    check(st == LSEC_OK && memcmp(s, s_ref, send_bytes) == 0, "pack_send bf16 N=4 B=9 H=8 D=128 (bit-exact)");

    /* the oracle's packed buffer as a receive buffer: unpack + combine, unpack */
    void* d_r = dev_copy(s_ref, send_bytes);
    void* d_y = NULL;
    float* d_L = NULL;
    HIP_OK(hipMalloc(&d_y, sizeof(uint16_t) * (size_t)(B * Hl * D)));
    HIP_OK(hipMalloc((void**)&d_L, sizeof(float) * (size_t)(B * Hl)));
    st = lsec_unpack_combine(d_r, N, B, Hl, D, LSEC_BF16, LSEC_BASE_E, d_y, d_L, NULL);
    HIP_OK(hipDeviceSynchronize());
    uint16_t* y = malloc(sizeof(uint16_t) * (size_t)(B * Hl * D));
    float* L = malloc(sizeof(float) * (size_t)(B * Hl));
    HIP_OK(hipMemcpy(y, d_y, sizeof(uint16_t) * (size_t)(B * Hl * D), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(L, d_L, sizeof(float) * (size_t)(B * Hl), hipMemcpyDeviceToHost));
    double* y_ref = malloc(sizeof(double) * (size_t)(B * Hl * D));
    double* L_ref = malloc(sizeof(double) * (size_t)(B * Hl));
    oracle_unpack_combine(s_ref, LSEC_BF16, N, B, Hl, D, 0, y_ref, L_ref);
    uint16_t* uo_ref = malloc(sizeof(uint16_t) * (size_t)(N * B * Hl * D));
    float* ul_ref = malloc(sizeof(float) * (size_t)(N * B * Hl));
    oracle_unpack(s_ref, N, B, Hl, D, 2, uo_ref, ul_ref);
    check(st == LSEC_OK && close_enough(y, LSEC_BF16, y_ref, B * Hl * D,
                                        max_abs(uo_ref, LSEC_BF16, N * B * Hl * D), L, L_ref,
                                        B * Hl),
          "unpack_combine bf16 on the oracle's packed buffer");

    void* d_uo = NULL;
    float* d_ul = NULL;
    HIP_OK(hipMalloc(&d_uo, sizeof(uint16_t) * (size_t)(N * B * Hl * D)));
    HIP_OK(hipMalloc((void**)&d_ul, sizeof(float) * (size_t)(N * B * Hl)));
    st = lsec_unpack(d_r, N, B, Hl, D, LSEC_BF16, d_uo, d_ul, NULL);
    HIP_OK(hipDeviceSynchronize());
    uint16_t* uo = malloc(sizeof(uint16_t) * (size_t)(N * B * Hl * D));
    float* ul = malloc(sizeof(float) * (size_t)(N * B * Hl));
    HIP_OK(hipMemcpy(uo, d_uo, sizeof(uint16_t) * (size_t)(N * B * Hl * D), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ul, d_ul, sizeof(float) * (size_t)(N * B * Hl), hipMemcpyDeviceToHost));
    check(st == LSEC_OK && memcmp(uo, uo_ref, sizeof(uint16_t) * (size_t)(N * B * Hl * D)) == 0 &&
              memcmp(ul, ul_ref, sizeof(float) * (size_t)(N * B * Hl)) == 0,
          "unpack bf16 (bit-exact)");
    HIP_OK(hipFree(d_o));
    HIP_OK(hipFree(d_l));
    HIP_OK(hipFree(d_s));
    HIP_OK(hipFree(d_r));
    HIP_OK(hipFree(d_y));
    HIP_OK(hipFree(d_L));
    HIP_OK(hipFree(d_uo));
    HIP_OK(hipFree(d_ul));
    free(o), free(l), free(s), free(s_ref), free(y), free(L), free(y_ref), free(L_ref);
    free(uo_ref), free(ul_ref), free(uo), free(ul);
}

/* Planes padded to T tokens; the valid count (query_start_loc[2] = 27) is in
 * device memory. Tokens [0, 27) match the oracle; the padding rows keep the
 * 0xff bytes the output was filled with. */
static void valid_count_case(void) {
    const int64_t N = 4, T = 40, Tv = 27, H = 4, D = 128, rows = T * H, n_out = N * rows * D;
    const int32_t qsl[3] = {0, 10, (int32_t)Tv};
    uint16_t* o = malloc(sizeof(uint16_t) * (size_t)n_out);
    float* l = malloc(sizeof(float) * (size_t)(N * rows));
    draw(35, OUT_BF16, n_out, N * rows, o, l, -5.0, 15.0);
    void* d_o = dev_copy(o, sizeof(uint16_t) * (size_t)n_out);
    void* d_l = dev_copy(l, sizeof(float) * (size_t)(N * rows));
    void* d_q = dev_copy(qsl, sizeof(qsl));
    void* d_y = NULL;
    float* d_L = NULL;
    HIP_OK(hipMalloc(&d_y, sizeof(uint16_t) * (size_t)(rows * D)));
    HIP_OK(hipMalloc((void**)&d_L, sizeof(float) * (size_t)rows));
    HIP_OK(hipMemset(d_y, 0xff, sizeof(uint16_t) * (size_t)(rows * D)));
    HIP_OK(hipMemset(d_L, 0xff, sizeof(float) * (size_t)rows));
    const int st = lsec_combine_planes_valid(d_o, rows * D, (const float*)d_l, rows, N, T, H, D,
                                             LSEC_BF16, LSEC_BASE_E, (const int32_t*)d_q, 2, d_y,
                                             d_L, NULL);
    HIP_OK(hipDeviceSynchronize());
    uint16_t* y = malloc(sizeof(uint16_t) * (size_t)(rows * D));
    float* L = malloc(sizeof(float) * (size_t)rows);
    HIP_OK(hipMemcpy(y, d_y, sizeof(uint16_t) * (size_t)(rows * D), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(L, d_L, sizeof(float) * (size_t)rows, hipMemcpyDeviceToHost));
    /* the first Tv tokens of each plane, gathered for the oracle */
    const int64_t vrows = Tv * H;
    uint16_t* ov = malloc(sizeof(uint16_t) * (size_t)(N * vrows * D));
    float* lv = malloc(sizeof(float) * (size_t)(N * vrows));
    for (int64_t n = 0; n < N; ++n) {
        memcpy(ov + n * vrows * D, o + n * rows * D, sizeof(uint16_t) * (size_t)(vrows * D));
        memcpy(lv + n * vrows, l + n * rows, sizeof(float) * (size_t)vrows);
    }
    double* y_ref = malloc(sizeof(double) * (size_t)(vrows * D));
    double* L_ref = malloc(sizeof(double) * (size_t)vrows);
    oracle_lse_combine(ov, LSEC_BF16, lv, N, Tv, H, D, 0, y_ref, L_ref);
    int untouched = 1;
    for (int64_t i = vrows * D; i < rows * D; ++i) untouched &= y[i] == 0xffff;
    const unsigned char* Lb = (const unsigned char*)(L + vrows);
    for (size_t i = 0; i < sizeof(float) * (size_t)(rows - vrows); ++i) untouched &= Lb[i] == 0xff;
    check(st == LSEC_OK && untouched &&
              close_enough(y, LSEC_BF16, y_ref, vrows * D, max_abs(ov, LSEC_BF16, N * vrows * D), L,
                           L_ref, vrows),
          "combine_planes_valid bf16 N=4 T=40 Tv=27 (count on device)");
    HIP_OK(hipFree(d_o));
    HIP_OK(hipFree(d_l));
    HIP_OK(hipFree(d_q));
    HIP_OK(hipFree(d_y));
    HIP_OK(hipFree(d_L));
    free(o), free(l), free(y), free(L), free(ov), free(lv), free(y_ref), free(L_ref);
}

/* A combining call's results [rows, D] (+ [rows]) copied back and checked. */
static int fetch_and_check(void* d_y, float* d_L, int64_t rows, int64_t D, int res_dtype,
                           const double* y_ref, const double* L_ref, double M) {
    const size_t ybytes = (size_t)(rows * D) * (res_dtype == LSEC_FP32 ? 4 : 2);
    void* y = malloc(ybytes);
    float* L = malloc(sizeof(float) * (size_t)rows);
    HIP_OK(hipMemcpy(y, d_y, ybytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(L, d_L, sizeof(float) * (size_t)rows, hipMemcpyDeviceToHost));
    const int ok = close_enough(y, res_dtype, y_ref, rows * D, M, L, L_ref, rows);
    free(y), free(L);
    return ok;
}

static void merge_case(int token_dim) {
    const int64_t N = 4, A = 13, C = 6, D = 128, rows = A * C, n_out = N * rows * D;
    uint16_t* o = malloc(sizeof(uint16_t) * (size_t)n_out);
    float* l = malloc(sizeof(float) * (size_t)(N * rows));
    draw(50 + (uint32_t)token_dim, OUT_BF16, n_out, N * rows, o, l, -5.0, 15.0);
    void* d_o = dev_copy(o, sizeof(uint16_t) * (size_t)n_out);
    void* d_l = dev_copy(l, sizeof(float) * (size_t)(N * rows));
    void* d_y = NULL;
    float* d_L = NULL;
    HIP_OK(hipMalloc(&d_y, sizeof(uint16_t) * (size_t)(rows * D)));
    HIP_OK(hipMalloc((void**)&d_L, sizeof(float) * (size_t)rows));
    const int st = lsec_merge(d_o, (const float*)d_l, N, A, C, D, token_dim, LSEC_BF16,
                              LSEC_BASE_E, d_y, d_L, NULL);
    HIP_OK(hipDeviceSynchronize());
    double* y_ref = malloc(sizeof(double) * (size_t)(rows * D));
    double* L_ref = malloc(sizeof(double) * (size_t)rows);
    oracle_merge(o, LSEC_BF16, l, N, A, C, D, token_dim, 0, y_ref, L_ref);
    check(st == LSEC_OK && fetch_and_check(d_y, d_L, rows, D, LSEC_BF16, y_ref, L_ref,
                                           max_abs(o, LSEC_BF16, n_out)),
          token_dim == 1 ? "merge bf16 N=4 A=13 C=6 D=128 token_dim 1"
                         : "merge bf16 N=4 A=13 C=6 D=128 token_dim 2 (token-major store)");
    HIP_OK(hipFree(d_o));
    HIP_OK(hipFree(d_l));
    HIP_OK(hipFree(d_y));
    HIP_OK(hipFree(d_L));
    free(o), free(l), free(y_ref), free(L_ref);
}

static void correct_case(void) {
    const int64_t N = 8, B = 21, H = 16, D = 512, rank = 5, rows = B * H;
    uint16_t* p = malloc(sizeof(uint16_t) * (size_t)(rows * D));
    float* l = malloc(sizeof(float) * (size_t)(N * rows));
    draw(60, OUT_BF16, rows * D, N * rows, p, l, -5.0, 15.0);
    void* d_p = dev_copy(p, sizeof(uint16_t) * (size_t)(rows * D));
    void* d_l = dev_copy(l, sizeof(float) * (size_t)(N * rows));
    void* d_y = NULL;
    float* d_L = NULL;
    HIP_OK(hipMalloc(&d_y, sizeof(uint16_t) * (size_t)(rows * D)));
    HIP_OK(hipMalloc((void**)&d_L, sizeof(float) * (size_t)rows));
    const int st = lsec_correct_partial((const float*)d_l, N, rank, d_p, B, H, D, LSEC_BF16,
                                        LSEC_BASE_2, d_y, d_L, NULL);
    HIP_OK(hipDeviceSynchronize());
    double* y_ref = malloc(sizeof(double) * (size_t)(rows * D));
    double* L_ref = malloc(sizeof(double) * (size_t)rows);
    oracle_correct_partial(l, N, rank, p, LSEC_BF16, B, H, D, 1, y_ref, L_ref);
    check(st == LSEC_OK && fetch_and_check(d_y, d_L, rows, D, LSEC_BF16, y_ref, L_ref,
                                           max_abs(p, LSEC_BF16, rows * D)),
          "correct_partial bf16 N=8 B=21 H=16 D=512 rank 5 base 2");
    HIP_OK(hipFree(d_p));
    HIP_OK(hipFree(d_l));
    HIP_OK(hipFree(d_y));
    HIP_OK(hipFree(d_L));
    free(p), free(l), free(y_ref), free(L_ref);
}

/* Planes of Tmax tokens of which the first T are combined (strided planes). */
static void planes_case(void) {
    const int64_t N = 4, Tmax = 50, T = 33, H = 4, D = 256, prow = Tmax * H, rows = T * H;
    uint16_t* o = malloc(sizeof(uint16_t) * (size_t)(N * prow * D));
    float* l = malloc(sizeof(float) * (size_t)(N * prow));
    draw(70, OUT_F16, N * prow * D, N * prow, o, l, 0.0, 20.0);
    void* d_o = dev_copy(o, sizeof(uint16_t) * (size_t)(N * prow * D));
    void* d_l = dev_copy(l, sizeof(float) * (size_t)(N * prow));
    void* d_y = NULL;
    float* d_L = NULL;
    HIP_OK(hipMalloc(&d_y, sizeof(uint16_t) * (size_t)(rows * D)));
    HIP_OK(hipMalloc((void**)&d_L, sizeof(float) * (size_t)rows));
    const int st = lsec_combine_planes(d_o, prow * D, (const float*)d_l, prow, N, T, H, D,
                                       LSEC_FP16, LSEC_BASE_2, d_y, d_L, NULL);
    HIP_OK(hipDeviceSynchronize());
    uint16_t* ov = malloc(sizeof(uint16_t) * (size_t)(N * rows * D));
    float* lv = malloc(sizeof(float) * (size_t)(N * rows));
    for (int64_t n = 0; n < N; ++n) {
        memcpy(ov + n * rows * D, o + n * prow * D, sizeof(uint16_t) * (size_t)(rows * D));
        memcpy(lv + n * rows, l + n * prow, sizeof(float) * (size_t)rows);
    }
    double* y_ref = malloc(sizeof(double) * (size_t)(rows * D));
    double* L_ref = malloc(sizeof(double) * (size_t)rows);
    oracle_lse_combine(ov, LSEC_FP16, lv, N, T, H, D, 1, y_ref, L_ref);
    check(st == LSEC_OK && fetch_and_check(d_y, d_L, rows, D, LSEC_FP16, y_ref, L_ref,
                                           max_abs(ov, LSEC_FP16, N * rows * D)),
          "combine_planes fp16 N=4 T=33 of 50 H=4 D=256 base 2");
    HIP_OK(hipFree(d_o));
    HIP_OK(hipFree(d_l));
    HIP_OK(hipFree(d_y));
    HIP_OK(hipFree(d_L));
    free(o), free(l), free(ov), free(lv), free(y_ref), free(L_ref);
}

/* More send rows than the pack's persistent grid takes in one pass: 1025
 * tiles of 64 rows, the last one partly filled. */
static void pack_walk_case(void) {
    const int64_t N = 4, B = 4099, H = 16, D = 128, rows = B * H;
    const int64_t W = D + lsec_pack_dim(LSEC_BF16);
    uint16_t* o = malloc(sizeof(uint16_t) * (size_t)(rows * D));
    float* l = malloc(sizeof(float) * (size_t)rows);
    draw(80, OUT_BF16, rows * D, rows, o, l, -5.0, 15.0);
    const size_t send_bytes = sizeof(uint16_t) * (size_t)(rows * W);
    void* d_o = dev_copy(o, sizeof(uint16_t) * (size_t)(rows * D));
    void* d_l = dev_copy(l, sizeof(float) * (size_t)rows);
    void* d_s = NULL;
    HIP_OK(hipMalloc(&d_s, send_bytes));
    const int st = lsec_pack_send(d_o, (const float*)d_l, N, B, H, D, LSEC_BF16, d_s, NULL);
    HIP_OK(hipDeviceSynchronize());
    uint16_t* s = malloc(send_bytes);
    uint16_t* s_ref = malloc(send_bytes);
    HIP_OK(hipMemcpy(s, d_s, send_bytes, hipMemcpyDeviceToHost));
    oracle_pack_send(o, l, N, B, H, D, 2, s_ref);
    check(st == LSEC_OK && memcmp(s, s_ref, send_bytes) == 0 &&
              strcmp(lsec_pack_path(N, B, H, D, LSEC_BF16, 1, 16), "pack_pipe_kernel") == 0,
          "pack_send bf16 N=4 B=4099 H=16 D=128, 1025 tiles (bit-exact)");
    HIP_OK(hipFree(d_o));
    HIP_OK(hipFree(d_l));
    HIP_OK(hipFree(d_s));
    free(o), free(l), free(s), free(s_ref);
}

static void diagnostics_cases(void) {
    check(strcmp(lsec_combine_path(16, 16384, 32, 128, LSEC_BF16, 0, 1),
                 "combine_tiled_kernel S=16") == 0 &&
              strcmp(lsec_combine_path(8, 2048, 8, 128, LSEC_BF16, 1, 1), "combine_span_kernel") == 0 &&
              strcmp(lsec_pack_path(8, 2048, 64, 128, LSEC_BF16, 1, 4), "pack_rows_kernel") == 0 &&
              strcmp(lsec_pack_path(8, 2048, 60, 128, LSEC_BF16, 1, 16), "none") == 0,
          "path diagnostics");
    int ok = 1;
    for (int code = LSEC_OK; code <= LSEC_ERR_RANK; ++code) {
        const char* a = lsec_status_string(code);
        ok &= a != NULL && strlen(a) > 0;
        for (int other = LSEC_OK; other < code; ++other) ok &= strcmp(a, lsec_status_string(other)) != 0;
    }
    ok &= lsec_status_string(12345) != NULL;
    check(ok, "a distinct status string for every status");
}

static void error_cases(void) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, 4096));
    /* each call is rejected before anything is enqueued */
    check(lsec_combine(d, (const float*)d, 2, 1, 1, 8, 7, LSEC_BASE_E, d, NULL, NULL) == LSEC_ERR_DTYPE,
          "unknown dtype -> LSEC_ERR_DTYPE");
    check(lsec_pack_send(d, (const float*)d, 3, 2, 8, 16, LSEC_BF16, d, NULL) == LSEC_ERR_DIVISIBILITY,
          "H % N != 0 -> LSEC_ERR_DIVISIBILITY");
    check(lsec_pack_send(d, (const float*)d, 2, 2, 8, 16, LSEC_BF16 | LSEC_OUT_FP32, d, NULL) ==
              LSEC_ERR_DTYPE,
          "fp32 result on a layout call -> LSEC_ERR_DTYPE");
    check(lsec_combine((const char*)d + 1, (const float*)d, 2, 1, 1, 8, LSEC_BF16, LSEC_BASE_E, d,
                       NULL, NULL) == LSEC_ERR_ALIGNMENT,
          "odd address -> LSEC_ERR_ALIGNMENT");
    check(strlen(lsec_status_string(LSEC_ERR_SHAPE)) > 0 && lsec_pack_dim(LSEC_FP32) == 1,
          "status strings and pack dims");
    check(lsec_merge(d, (const float*)d, 2, 1, 1, 8, 3, LSEC_BF16, LSEC_BASE_E, d, NULL, NULL) ==
              LSEC_ERR_TOKEN_DIM,
          "token_dim 3 -> LSEC_ERR_TOKEN_DIM");
    check(lsec_correct_partial((const float*)d, 2, 2, d, 1, 1, 8, LSEC_BF16, LSEC_BASE_E, d, NULL,
                               NULL) == LSEC_ERR_RANK,
          "rank N -> LSEC_ERR_RANK");
    HIP_OK(hipFree(d));
}

int main(void) {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
        fprintf(stderr, "c_abi_check: no usable GPU\n");
        return 2;
    }
    printf("liblsec version %d\n", lsec_version());
    combine_case("combine bf16 N=8 B=37 H=5 D=128 base e + LSE (tiled)", 31, 8, 37, 5, 128,
                 LSEC_BF16, LSEC_BASE_E, 0);
    combine_case("combine fp16 N=3 B=20 H=3 D=64 base 2 + LSE (row kernel)", 32, 3, 20, 3, 64,
                 LSEC_FP16, LSEC_BASE_2, 0);
    combine_case("combine bf16 -> fp32 N=4 B=33 H=4 D=256 base e + LSE", 33, 4, 33, 4, 256,
                 LSEC_BF16, LSEC_BASE_E, 1);
    packed_case();
    pack_walk_case();
    valid_count_case();
    planes_case();
    merge_case(1);
    merge_case(2);
    correct_case();
    diagnostics_cases();
    error_cases();
    printf("c_abi_check: %s\n", failures ? "FAILED" : "ok");
    return failures ? 1 : 0;
}
