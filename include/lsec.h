/*
 * lsec.h -- C ABI of the LSE-weighted combine library (liblsec.so), gfx950.
 *
 * The operations are those of the page "vllm.v1.attention.ops.dcp_alltoall"
 * (lsec_merge: of the page "vllm_ascend/attention/context_parallel/sfa_cp.py"):
 *  - lsec_combine        : `_lse_weighted_combine` (merge N partial attention
 *                          outputs by their log-sum-exp weights);
 *  - lsec_pack_send      : `_dcp_a2a_pack_send` inside `dcp_a2a_lse_reduce`
 *                          (output + fp32 LSE packed into one output-dtype
 *                          buffer, one plane per destination rank);
 *  - lsec_unpack_combine : `_dcp_a2a_unpack_combine` (the receive side: read
 *                          the packed planes and combine them);
 *  - lsec_unpack         : the layout half of that step alone;
 *  - lsec_pack_dim       : `_dcp_a2a_lse_pack_dim`.
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers unless stated otherwise. Tensors are dense,
 *    row-major, last dimension fastest, with no padding between rows.
 *  - The caller owns and allocates every buffer; the library never allocates,
 *    frees or synchronises. Work is enqueued on `stream` (a hipStream_t; NULL
 *    means the null stream) and the call returns at once.
 *  - Elements of `outputs`, `partial`, `send`, `recv` are bf16, fp16 or fp32
 *    (selected by `dtype`) and must be aligned to their size; LSE arrays are
 *    fp32 and must be 4-byte aligned. `out` holds elements of the input dtype,
 *    or fp32 when the combining calls (lsec_combine, lsec_merge,
 *    lsec_unpack_combine, lsec_correct_partial) get `dtype | LSEC_OUT_FP32`.
 *    Faster kernels are chosen when the buffers are 16-byte aligned (separate
 *    layout) or 4-byte aligned (packed layout) and a row is whole 16-byte
 *    chunks that fit 256 lanes (D a multiple of 8 up to 2048 for 16-bit
 *    elements, of 4 up to 1024 for fp32); other cases take a general path
 *    with the same results.
 *  - Every argument is checked before anything is enqueued; on an error
 *    nothing is enqueued and a status other than LSEC_OK is returned. A
 *    pointer may be NULL only when the array it names has no elements.
 *  - Input and output buffers must not overlap.
 *  - Arithmetic: fp32 accumulation; 16-bit outputs are rounded to nearest
 *    even from fp32; the global LSE is fp32. NaN and +-inf shard LSEs
 *    count as -inf; a row whose shard LSEs are all non-finite yields a zero
 *    output and a -inf global LSE. Zero-weight shards are still multiplied, so
 *    a NaN in any shard's output propagates to the combined output.
 */
#ifndef LSEC_H
#define LSEC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    LSEC_OK = 0,
    LSEC_ERR_NULL = 1,         /* a required pointer is NULL */
    LSEC_ERR_SHAPE = 2,        /* N < 1, B < 0, H < 1, D < 1, or a size overflows int64 */
    LSEC_ERR_DIVISIBILITY = 3, /* H is not a multiple of N (pack_send) */
    LSEC_ERR_DTYPE = 4,        /* unknown dtype, or LSEC_OUT_FP32 on a layout-only call */
    LSEC_ERR_ALIGNMENT = 5,    /* a pointer is not aligned to its element size */
    LSEC_ERR_BASE = 6,         /* base is neither LSEC_BASE_E nor LSEC_BASE_2 */
    LSEC_ERR_LAUNCH = 7,       /* the HIP runtime rejected the kernel launch */
    LSEC_ERR_TOKEN_DIM = 8,    /* token_dim is neither 1 nor 2 (lsec_merge) */
    LSEC_ERR_RANK = 9          /* rank outside [0, N) (lsec_correct_partial) */
};

/* Element types of the attention outputs. */
enum { LSEC_BF16 = 0, LSEC_FP16 = 1, LSEC_FP32 = 2 };

/*
 * OR'ed into the `dtype` of a combining call: write the result in fp32 even
 * for bf16 / fp16 inputs. The page's CPU function `_lse_weighted_combine`
 * multiplies the 16-bit outputs by fp32 weights, so its result is promoted to
 * fp32; without the flag the result is rounded back to the input dtype (what
 * the exchange paths return). fp32 inputs always give fp32 results.
 */
enum { LSEC_OUT_FP32 = 256 };

/* Base of the log-sum-exp values (`is_lse_base_on_e` true / false). */
enum { LSEC_BASE_E = 0, LSEC_BASE_2 = 1 };

/*
 * lsec_pack_dim -- number of output-dtype elements that carry one fp32 LSE in
 * a packed row: P = 4 / sizeof(element) = 2 for bf16 and fp16, 1 for fp32.
 * Returns -1 for an unknown dtype (the LSEC_OUT_FP32 flag included).
 * (`_dcp_a2a_lse_pack_dim`; its body is not on the page, this is the reading
 * that makes the packed row D + P elements wide.)
 */
int lsec_pack_dim(int dtype);

/*
 * lsec_combine -- `_lse_weighted_combine`.
 *   outputs : [N, B, H, D] dtype   partial attention output of each shard
 *   lses    : [N, B, H]    fp32    per-shard log-sum-exp, base `base`
 *   out     : [B, H, D]    dtype   combined output (written; fp32 with
 *                                  LSEC_OUT_FP32 or fp32 inputs)
 *   out_lse : [B, H]       fp32    global LSE (written), or NULL to skip it
 *                                  (`return_lse` false)
 * Per (b, h) row: l'_n = -inf if l_n is NaN or +-inf; m = max_n l'_n (0 if
 * that is -inf); w_n = exp(l'_n - m) or 2^(l'_n - m); S = sum_n w_n;
 * out = sum_n outputs_n * w_n / max(S, 1e-10); out_lse = ln S + m or
 * log2 S + m. N = 1 with a finite LSE returns its input unchanged, bit for
 * bit (-0 and subnormals included), and its LSE as the global LSE.
 * Errors: NULL, SHAPE, DTYPE, BASE, ALIGNMENT, LAUNCH.
 */
int lsec_combine(const void* outputs, const float* lses, int64_t N, int64_t B, int64_t H,
                 int64_t D, int dtype, int base, void* out, float* out_lse, void* stream);

/*
 * lsec_combine_planes -- lsec_combine over planes that are the leading rows of
 * longer ones: the local combine of the fused direct all-to-all of the page
 * "vllm.v1.attention.ops.dcp" (`DirectDCPA2AWorkspace.lse_reduce`), whose
 * receive buffers hold, per ubatch and slot, W planes
 * [W, T_max, H_r, D] (+ LSEs [W, T_max, H_r]) of which the first T tokens
 * belong to the current step. The caller picks the ubatch and slot by the
 * base pointers; the library reads nothing beyond the first T tokens.
 *   outputs          : plane n = the T * H * D elements at
 *                      outputs + n * plane_stride (dtype)
 *   plane_stride     : elements between planes, >= T * H * D (T_max * H * D)
 *   lses             : plane n = the T * H fp32 at lses + n * lse_plane_stride
 *   lse_plane_stride : >= T * H (T_max * H)
 *   out, out_lse     : [T, H, D], [T, H] exactly as in lsec_combine
 * With plane_stride = T*H*D and lse_plane_stride = T*H this is lsec_combine.
 * The fast kernels also need plane_stride * sizeof(element) to be a multiple
 * of 16 bytes; other strides take the general path with the same results.
 * Errors: NULL, SHAPE (also a stride below its plane's size), DTYPE, BASE,
 * ALIGNMENT, LAUNCH.
 */
int lsec_combine_planes(const void* outputs, int64_t plane_stride, const float* lses,
                        int64_t lse_plane_stride, int64_t N, int64_t T, int64_t H, int64_t D,
                        int dtype, int base, void* out, float* out_lse, void* stream);

/*
 * lsec_combine_planes_valid -- lsec_combine_planes whose count of valid tokens
 * lives in device memory: the `query_start_loc` argument of the same page's
 * `DirectDCPA2AWorkspace.lse_reduce` (that op's body is not given; the reading
 * taken here is that its masking marks the tokens past the last request as
 * padding). query_start_loc holds the num_reqs + 1 cumulative token offsets
 * of the step's requests (int32, device memory); the kernels read
 * Tv = query_start_loc[num_reqs], clamped to [0, T], and combine tokens
 * [0, Tv) exactly as lsec_combine_planes does. Tokens [Tv, T) are padding:
 * their rows of out and out_lse are not written and their planes are not
 * read. T is the token capacity of out (a padded batch, e.g. a captured
 * graph's size), so the host never has to read Tv. The per-request sequence
 * lengths of that op are not needed: a shard with no keys for a request
 * carries a NaN or infinite LSE, which the combine already drops.
 *   query_start_loc : int32 [num_reqs + 1], device memory, 4-byte aligned;
 *                     only element num_reqs is read
 *   num_reqs        : >= 0
 *   other arguments : as lsec_combine_planes (T = the capacity)
 * Errors: as lsec_combine_planes; NULL also for a NULL query_start_loc when
 * T * H > 0, SHAPE for num_reqs < 0 or H >= 2^32, ALIGNMENT for a misaligned
 * query_start_loc.
 */
int lsec_combine_planes_valid(const void* outputs, int64_t plane_stride, const float* lses,
                              int64_t lse_plane_stride, int64_t N, int64_t T, int64_t H,
                              int64_t D, int dtype, int base, const int32_t* query_start_loc,
                              int64_t num_reqs, void* out, float* out_lse, void* stream);

/*
 * lsec_merge -- the merge of page "vllm_ascend/attention/context_parallel/
 * sfa_cp.py", `_merge_dcp_outputs_with_torch`: the combine of lsec_combine over
 * received planes whose token index is the first or the second of the two row
 * dimensions, written token-major (the merge's trailing `movedim`).
 *   outputs : [N, A, C, D] dtype   plane n = what rank n sent
 *   lses    : [N, A, C]    fp32
 *   token_dim == 1 (tokens are A, e.g. token-sharded exchange):
 *       out [A, C, D], out_lse [A, C]     -- identical to lsec_combine(B=A, H=C)
 *   token_dim == 2 (tokens are C, e.g. head-sharded exchange [N, Hl, T, D]):
 *       out [C, A, D], out_lse [C, A]     -- row (a, c) is stored at (c, a)
 * The page's merge is base e and returns no LSE; `base` and `out_lse` extend
 * it exactly as in lsec_combine (out_lse may be NULL).
 * Errors: TOKEN_DIM, NULL, SHAPE, DTYPE, BASE, ALIGNMENT, LAUNCH.
 */
int lsec_merge(const void* outputs, const float* lses, int64_t N, int64_t A, int64_t C,
               int64_t D, int token_dim, int dtype, int base, void* out, float* out_lse,
               void* stream);

/*
 * lsec_correct_partial -- the local step of the LSE all-gather + output
 * reduce-scatter / all-reduce strategies that the page
 * "vllm.v1.attention.ops.dcp" selects in `MLADCPManager` (`cp_lse_ag_out_rs`,
 * `cp_lse_ag_out_ar`; only their names are shown, so this is a reading):
 *   lses    : [N, B, H]  fp32   every shard's LSE (after the all-gather)
 *   rank    : r in [0, N)       this rank's shard
 *   partial : [B, H, D]  dtype  this rank's partial output
 *   out     : [B, H, D]  dtype  partial * w_r / max(S, 1e-10) (written; fp32
 *                               with LSEC_OUT_FP32, e.g. to sum in fp32)
 *   out_lse : [B, H]     fp32   global LSE (written), or NULL
 * with w_r and S exactly as in lsec_combine, so the sum of `out` over the N
 * ranks (what the reduce-scatter / all-reduce computes) is the combine.
 * Errors: RANK, NULL, SHAPE, DTYPE, BASE, ALIGNMENT, LAUNCH.
 */
int lsec_correct_partial(const float* lses, int64_t N, int64_t rank, const void* partial,
                         int64_t B, int64_t H, int64_t D, int dtype, int base, void* out,
                         float* out_lse, void* stream);

/*
 * lsec_pack_send -- `_dcp_a2a_pack_send`.
 *   attn_out : [B, H, D]           dtype  this rank's partial attention output
 *   attn_lse : [B, H]              fp32   its log-sum-exp
 *   send     : [N, B, H/N, D + P]  dtype  packed send buffer (written),
 *                                         P = lsec_pack_dim(dtype)
 * Plane r holds heads [r*H/N, (r+1)*H/N): the chunk an all-to-all delivers to
 * rank r. In each packed row, elements 0..D-1 are the output row, and the P
 * tail elements hold the four bytes of the fp32 LSE in memory order (16-bit:
 * element D = bits 0..15, element D+1 = bits 16..31; fp32: element D is the
 * LSE's own pattern). Pure bit moves (NaN payloads kept).
 * Errors: NULL, SHAPE, DIVISIBILITY (H % N != 0), DTYPE, ALIGNMENT, LAUNCH.
 */
int lsec_pack_send(const void* attn_out, const float* attn_lse, int64_t N, int64_t B, int64_t H,
                   int64_t D, int dtype, void* send, void* stream);

/*
 * lsec_unpack_combine -- `_dcp_a2a_unpack_combine`.
 *   recv    : [N, B, Hl, D + P] dtype  packed planes; plane n came from rank n
 *   out     : [B, Hl, D]        dtype  combined output (written; fp32 with
 *                                      LSEC_OUT_FP32 or fp32 inputs)
 *   out_lse : [B, Hl]           fp32   global LSE (written), or NULL
 * Equivalent to lsec_unpack followed by lsec_combine with H = Hl, in one pass.
 * Errors: NULL, SHAPE, DTYPE, BASE, ALIGNMENT, LAUNCH.
 */
int lsec_unpack_combine(const void* recv, int64_t N, int64_t B, int64_t Hl, int64_t D, int dtype,
                        int base, void* out, float* out_lse, void* stream);

/*
 * lsec_unpack -- the layout half of the receive step.
 *   recv    : [N, B, Hl, D + P] dtype
 *   outputs : [N, B, Hl, D]     dtype  (written)
 *   lses    : [N, B, Hl]        fp32   (written; the tail bits reinterpreted)
 * Pure bit moves; the inverse of lsec_pack_send's per-row layout.
 * Errors: NULL, SHAPE, DTYPE, ALIGNMENT, LAUNCH.
 */
int lsec_unpack(const void* recv, int64_t N, int64_t B, int64_t Hl, int64_t D, int dtype,
                void* outputs, float* lses, void* stream);

/*
 * lsec_combine_path -- diagnostics: the name of the kernel lsec_combine
 * (packed == 0, H = heads) or lsec_unpack_combine (packed != 0, H = heads per
 * rank, Hl) launches for these sizes and `dtype` (as passed to those calls),
 * given whether the buffers meet the fast alignment (aligned_buffers != 0: 16
 * bytes for outputs, recv and out). Returns a static string such as
 * "combine_tiled_kernel S=16", "combine_span_kernel", "combine_span32_kernel",
 * "combine_rows_kernel" or "combine_elems_kernel"; "none" when the arguments
 * launch nothing or are invalid. Touches no GPU state.
 */
const char* lsec_combine_path(int64_t N, int64_t B, int64_t H, int64_t D, int dtype, int packed,
                              int aligned_buffers);

/*
 * lsec_pack_path -- diagnostics: the name of the kernel lsec_pack_send
 * launches for these sizes and `dtype` (as passed to it; no LSEC_OUT_FP32),
 * given whether attn_out is 16-byte aligned (in_aligned != 0) and the
 * alignment of the send buffer in bytes (send_align: 16 or more, 4 to 15, or
 * less). Returns a static string: "pack_pipe_kernel" (whole 16-byte chunks
 * of D, 16-byte aligned buffers: rows assembled in LDS, a persistent grid),
 * "pack_rows_kernel" (a send buffer aligned to 4 bytes only),
 * "pack_elems_kernel" (any other), or "none" when the arguments are invalid.
 * Touches no GPU state.
 */
const char* lsec_pack_path(int64_t N, int64_t B, int64_t H, int64_t D, int dtype, int in_aligned,
                           int send_align);

/* Human-readable text for a status code (static storage; never NULL). */
const char* lsec_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int lsec_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LSEC_H */
