/*
 * oracle.c -- plain, slow, fp64 CPU reference for the LSE-weighted combine
 * and its pack / unpack layout.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg may load or call this code. The product path
 * (the HIP library and its Python binding) never does, and shares no code,
 * header, table or helper with it.
 *
 * Sources (the web pages this follows):
 *  - "vllm.v1.attention.ops.dcp_alltoall", function `_lse_weighted_combine`:
 *    the combine, step by step (sanitise, max, weights, NaN-weight guard,
 *    clamped normalisation, weighted sum, global LSE).
 *  - same page, function `dcp_a2a_lse_reduce`: the packed exchange buffer
 *    [N, B, H/N, D + P] in the output dtype, filled by `_dcp_a2a_pack_send`,
 *    moved by an all-to-all whose chunk r goes to rank r, and consumed by
 *    `_dcp_a2a_unpack_combine`.
 *
 * Readings where the pages leave a step open:
 *  - P (`_dcp_a2a_lse_pack_dim`) is the number of output elements that hold
 *    one fp32 LSE: 4 / sizeof(dtype) = 2 for bf16 and fp16, 1 for fp32.
 *  - The fp32 LSE occupies the P tail elements in memory order (its four
 *    bytes copied verbatim, little-endian on every target here).
 *  - Plane r of the send buffer holds heads [r*Hl, (r+1)*Hl) in order.
 *  - Arithmetic is fp64 throughout; inputs are converted exactly (every bf16,
 *    fp16 and fp32 value is a double). The combined output is returned
 *    unrounded, in fp64; the caller's result dtype (the input dtype, or the
 *    fp32 that the page's CPU function promotes bf16 / fp16 products to) only
 *    changes the tolerance of a comparison, not the oracle.
 *
 * Build: gcc -O2 -std=c11 (no fast-math: the NaN / inf tests must survive).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_BF16 = 0, ORACLE_F16 = 1, ORACLE_F32 = 2 };

/* Bytes per stored element of a dtype, or 0 for an unknown dtype. */
static int64_t elem_bytes(int dtype) {
    return dtype == ORACLE_BF16 || dtype == ORACLE_F16 ? 2 : dtype == ORACLE_F32 ? 4 : 0;
}

/* ---- exact storage-to-fp64 conversions ---- */

/* bf16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t h) {
    uint32_t x = (uint32_t)h << 16;
    float f;
    memcpy(&f, &x, 4);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0x1f) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -24);            /* subnormal: m * 2^-24 */
    else v = ldexp((double)(m | 0x400), e - 25);            /* (1024+m) * 2^(e-15-10) */
    return sign ? -v : v;
}

/* IEEE binary32: the bits reinterpreted as a float, then widened (exact). */
double oracle_f32_to_f64(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Element i of an array of stored elements of the given dtype, as fp64. */
static double load_elem(const void* base, int64_t i, int dtype) {
    if (dtype == ORACLE_F32) {
        uint32_t u;
        memcpy(&u, (const char*)base + 4 * i, 4);
        return oracle_f32_to_f64(u);
    }
    uint16_t h;
    memcpy(&h, (const char*)base + 2 * i, 2);
    return dtype == ORACLE_BF16 ? oracle_bf16_to_f64(h) : oracle_f16_to_f64(h);
}

/* Array form of the conversions above. Returns 0, or -1 on a bad dtype. */
int oracle_bits_to_f64(const void* bits, int dtype, int64_t n, double* out) {
    if (!elem_bytes(dtype)) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = load_elem(bits, i, dtype);
    return 0;
}

/* ---- the combine on fp64 planes ----
 *
 * o   : [N][R][D] partial outputs, R = independent (token, head) rows
 * lse : [N][R]    per-shard log-sum-exp (base e, or base 2 when base2 != 0)
 * y   : [R][D]    combined output
 * L   : [R]       global LSE (may be NULL)
 *
 * Follows `_lse_weighted_combine` one row at a time.
 */
void oracle_combine_f64(const double* o, const double* lse, int64_t N, int64_t R, int64_t D,
                        int base2, double* y, double* L) {
    for (int64_t r = 0; r < R; ++r) {
        double l[N > 0 ? N : 1];
        double w[N > 0 ? N : 1];
        /* NaN and +-inf shard LSEs become -inf. */
        for (int64_t n = 0; n < N; ++n) {
            double v = lse[n * R + r];
            l[n] = (isnan(v) || isinf(v)) ? -INFINITY : v;
        }
        /* max over shards; an all -inf max is replaced by 0. */
        double m = -INFINITY;
        for (int64_t n = 0; n < N; ++n)
            if (l[n] > m) m = l[n];
        if (m == -INFINITY) m = 0.0;
        /* weights exp(l - m) or 2^(l - m); a NaN weight becomes 0. */
        for (int64_t n = 0; n < N; ++n) {
            w[n] = base2 ? pow(2.0, l[n] - m) : exp(l[n] - m);
            if (isnan(w[n])) w[n] = 0.0;
        }
        /* sum of weights (in shard order); normalise by the sum clamped at 1e-10. */
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n) s += w[n];
        double denom = s < 1e-10 ? 1e-10 : s;
        double wn[N > 0 ? N : 1];
        for (int64_t n = 0; n < N; ++n) wn[n] = w[n] / denom;
        /* weighted sum over shards. */
        for (int64_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) acc += o[(n * R + r) * D + d] * wn[n];
            y[r * D + d] = acc;
        }
        /* global LSE from the unclamped sum. */
        if (L) L[r] = (base2 ? log2(s) : log(s)) + m;
    }
}

/* ---- the combine on storage-typed inputs ----
 *
 * outputs : [N][B][H][D] bf16, fp16 or fp32 bits;  lses : [N][B][H] fp32
 * y : [B][H][D] fp64;  L : [B][H] fp64 or NULL.
 * Converts each row's inputs exactly to fp64, then runs oracle_combine_f64 on
 * that row. Returns 0, or -1 on a bad argument.
 */
int oracle_lse_combine(const void* outputs, int dtype, const float* lses, int64_t N,
                       int64_t B, int64_t H, int64_t D, int base2, double* y, double* L) {
    if (N < 1 || B < 0 || H < 1 || D < 1 || !elem_bytes(dtype)) return -1;
    int64_t R = B * H;
    double* ob = (double*)malloc(sizeof(double) * (size_t)(N * D + N));
    if (!ob) return -2;
    double* lb = ob + N * D;
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t n = 0; n < N; ++n) {
            lb[n] = (double)lses[n * R + r];
            for (int64_t d = 0; d < D; ++d)
                ob[n * D + d] = load_elem(outputs, (n * R + r) * D + d, dtype);
        }
        oracle_combine_f64(ob, lb, N, 1, D, base2, &y[r * D], L ? &L[r] : 0);
    }
    free(ob);
    return 0;
}

/* ---- the local step of an LSE all-gather + output reduce-scatter ----
 *
 * The page "vllm.v1.attention.ops.dcp" names the strategies
 * `cp_lse_ag_out_rs` and `cp_lse_ag_out_ar` without showing them. Reading:
 * every rank holds the gathered LSEs of all N shards and its own partial
 * output o_r; it scales o_r by shard r's normalised weight from
 * `_lse_weighted_combine` (steps sanitise, max, weights, NaN guard, clamped
 * normalisation), and the collective then sums the scaled partials over the
 * ranks, which gives the combine. L is the global LSE of the same function.
 *   lses [N][B][H] fp32; partial [B][H][D] bf16/fp16/fp32 bits of rank `rank`
 *   y [B][H][D] fp64 = partial * w_rank / max(S, 1e-10);  L [B][H] or NULL.
 */
int oracle_correct_partial(const float* lses, int64_t N, int64_t rank, const void* partial,
                           int dtype, int64_t B, int64_t H, int64_t D, int base2, double* y,
                           double* L) {
    if (N < 1 || rank < 0 || rank >= N || B < 0 || H < 1 || D < 1 || !elem_bytes(dtype))
        return -1;
    const int64_t R = B * H;
    double* l = (double*)malloc(sizeof(double) * (size_t)N);
    if (!l) return -2;
    for (int64_t r = 0; r < R; ++r) {
        /* NaN and +-inf shard LSEs become -inf. */
        for (int64_t n = 0; n < N; ++n) {
            double v = (double)lses[n * R + r];
            l[n] = (isnan(v) || isinf(v)) ? -INFINITY : v;
        }
        /* max over shards; an all -inf max is replaced by 0. */
        double m = -INFINITY;
        for (int64_t n = 0; n < N; ++n)
            if (l[n] > m) m = l[n];
        if (m == -INFINITY) m = 0.0;
        /* weights; a NaN weight becomes 0; the sum in shard order. */
        double s = 0.0, wr = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double w = base2 ? pow(2.0, l[n] - m) : exp(l[n] - m);
            if (isnan(w)) w = 0.0;
            s += w;
            if (n == rank) wr = w;
        }
        const double wn = wr / (s < 1e-10 ? 1e-10 : s);
        for (int64_t d = 0; d < D; ++d) y[r * D + d] = load_elem(partial, r * D + d, dtype) * wn;
        if (L) L[r] = (base2 ? log2(s) : log(s)) + m;
    }
    free(l);
    return 0;
}

/* ---- the token-major merge ----
 *
 * Follows `_merge_dcp_outputs_with_torch` on the page
 * "vllm_ascend/attention/context_parallel/sfa_cp.py": the received planes
 * outputs [N][A][C][D] and lses [N][A][C] are combined per (a, c) row, and the
 * result is laid out token-major (its closing `movedim`): token_dim 1 keeps
 * y [A][C][D]; token_dim 2 stores row (a, c) at (c, a), y [C][A][D]. L is laid
 * out the same way ([A][C] or [C][A]). The combine itself is the one above.
 */
int oracle_merge(const void* outputs, int dtype, const float* lses, int64_t N, int64_t A,
                 int64_t C, int64_t D, int token_dim, int base2, double* y, double* L) {
    if (N < 1 || A < 0 || C < 1 || D < 1 || (token_dim != 1 && token_dim != 2) ||
        !elem_bytes(dtype))
        return -1;
    const int64_t R = A * C;
    double* ob = (double*)malloc(sizeof(double) * (size_t)(N * D + N));
    if (!ob) return -2;
    double* lb = ob + N * D;
    for (int64_t a = 0; a < A; ++a)
        for (int64_t c = 0; c < C; ++c) {
            const int64_t r = a * C + c;                           /* input row */
            const int64_t o = token_dim == 1 ? r : c * A + a;      /* output row */
            for (int64_t n = 0; n < N; ++n) {
                lb[n] = (double)lses[n * R + r];
                for (int64_t d = 0; d < D; ++d)
                    ob[n * D + d] = load_elem(outputs, (n * R + r) * D + d, dtype);
            }
            oracle_combine_f64(ob, lb, N, 1, D, base2, &y[o * D], L ? &L[o] : 0);
        }
    free(ob);
    return 0;
}

/* ---- pack / unpack (pure byte moves) ----
 *
 * Elements are E = 2 (bf16, fp16) or 4 (fp32) bytes wide; P = 4 / E.
 * pack:   out [B][H][D] elements, lse [B][H] fp32
 *      -> send [N][B][Hl][D+P] elements, Hl = H / N:
 *         send[r][b][h][0:D]   = out[b][r*Hl + h][0:D]
 *         send[r][b][h][D:D+P] = the 4 bytes of lse[b][r*Hl + h]
 * unpack: recv [N][B][Hl][D+P] -> outputs [N][B][Hl][D], lses [N][B][Hl]
 *         (plane n of recv is what source rank n sent).
 */
int oracle_pack_dim(int elem_bytes) { return elem_bytes > 0 && elem_bytes <= 4 ? 4 / elem_bytes : -1; }

int oracle_pack_send(const void* out, const float* lse, int64_t N, int64_t B, int64_t H,
                     int64_t D, int64_t E, void* send) {
    if (N < 1 || B < 0 || H < 1 || D < 1 || H % N != 0 || (E != 2 && E != 4)) return -1;
    const int64_t P = 4 / E, Hl = H / N, W = D + P;
    const char* o = (const char*)out;
    char* s = (char*)send;
    for (int64_t r = 0; r < N; ++r)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t h = 0; h < Hl; ++h) {
                const int64_t src = b * H + r * Hl + h;
                char* dst = s + ((r * B + b) * Hl + h) * W * E;
                for (int64_t d = 0; d < D; ++d) memcpy(dst + d * E, o + (src * D + d) * E, (size_t)E);
                memcpy(dst + D * E, &lse[src], 4);
            }
    return 0;
}

int oracle_unpack(const void* recv, int64_t N, int64_t B, int64_t Hl, int64_t D, int64_t E,
                  void* outputs, float* lses) {
    if (N < 1 || B < 0 || Hl < 1 || D < 1 || (E != 2 && E != 4)) return -1;
    const int64_t P = 4 / E, W = D + P, R = B * Hl;
    const char* rv = (const char*)recv;
    char* os = (char*)outputs;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t r = 0; r < R; ++r) {
            const char* src = rv + (n * R + r) * W * E;
            for (int64_t d = 0; d < D; ++d)
                memcpy(os + ((n * R + r) * D + d) * E, src + d * E, (size_t)E);
            memcpy(&lses[n * R + r], src + D * E, 4);
        }
    return 0;
}

/* unpack, then combine: recv [N][B][Hl][D+P] -> y [B][Hl][D] fp64, L [B][Hl]. */
int oracle_unpack_combine(const void* recv, int dtype, int64_t N, int64_t B, int64_t Hl,
                          int64_t D, int base2, double* y, double* L) {
    const int64_t E = elem_bytes(dtype);
    if (N < 1 || B < 0 || Hl < 1 || D < 1 || !E) return -1;
    const int64_t P = 4 / E, W = D + P, R = B * Hl;
    const char* rv = (const char*)recv;
    double* ob = (double*)malloc(sizeof(double) * (size_t)(N * D + N));
    if (!ob) return -2;
    double* lb = ob + N * D;
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t n = 0; n < N; ++n) {
            const char* src = rv + (n * R + r) * W * E;
            float lf;
            memcpy(&lf, src + D * E, 4);
            lb[n] = (double)lf;
            for (int64_t d = 0; d < D; ++d) ob[n * D + d] = load_elem(src, d, dtype);
        }
        oracle_combine_f64(ob, lb, N, 1, D, base2, &y[r * D], L ? &L[r] : 0);
    }
    free(ob);
    return 0;
}

/* ---- the valid tokens of a padded step ----
 *
 * `DirectDCPA2AWorkspace.lse_reduce` on the page "vllm.v1.attention.ops.dcp"
 * takes the step's `seq_lens` and `query_start_loc`, but the page does not
 * show what the op does with them. Reading: `query_start_loc` holds the
 * num_reqs + 1 cumulative token offsets of the step's requests (entry i is
 * where request i's tokens start), so entry num_reqs is the number of real
 * tokens; the tokens from there up to the padded capacity T are padding and
 * get no result. The count is clamped to [0, T]. `seq_lens` changes nothing:
 * a shard that holds no key of a request reports a NaN or infinite LSE for
 * it, and the combine already drops such a shard.
 * Returns the count, or -1 on a bad argument.
 */
int64_t oracle_valid_tokens(const int32_t* query_start_loc, int64_t num_reqs, int64_t capacity) {
    if (!query_start_loc || num_reqs < 0 || capacity < 0) return -1;
    int64_t t = query_start_loc[num_reqs];
    if (t < 0) t = 0;
    if (t > capacity) t = capacity;
    return t;
}

/* The combine over the valid tokens of padded planes:
 * outputs [N][T][H][D] bf16, fp16 or fp32 bits, lses [N][T][H] fp32 (T = the
 * capacity); tokens [0, Tv) with Tv = oracle_valid_tokens(...) are combined
 * exactly as oracle_lse_combine does: y [Tv][H][D] fp64, L [Tv][H] or NULL.
 * *tv receives Tv. Returns 0, or -1 on a bad argument.
 */
int oracle_lse_combine_valid(const void* outputs, int dtype, const float* lses,
                             const int32_t* query_start_loc, int64_t num_reqs, int64_t N,
                             int64_t T, int64_t H, int64_t D, int base2, double* y, double* L,
                             int64_t* tv) {
    if (N < 1 || T < 0 || H < 1 || D < 1 || !elem_bytes(dtype) || !tv) return -1;
    const int64_t Tv = oracle_valid_tokens(query_start_loc, num_reqs, T);
    if (Tv < 0) return -1;
    *tv = Tv;
    const int64_t plane = T * H; /* rows per plane, padding included */
    double* ob = (double*)malloc(sizeof(double) * (size_t)(N * D + N));
    if (!ob) return -2;
    double* lb = ob + N * D;
    for (int64_t r = 0; r < Tv * H; ++r) {
        for (int64_t n = 0; n < N; ++n) {
            lb[n] = (double)lses[n * plane + r];
            for (int64_t d = 0; d < D; ++d)
                ob[n * D + d] = load_elem(outputs, (n * plane + r) * D + d, dtype);
        }
        oracle_combine_f64(ob, lb, N, 1, D, base2, &y[r * D], L ? &L[r] : 0);
    }
    free(ob);
    return 0;
}
