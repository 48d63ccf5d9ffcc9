// lsec.hip -- HIP kernels (gfx950) and the C ABI of liblsec.so.
//
// The operations are those of the page "vllm.v1.attention.ops.dcp_alltoall":
// `_lse_weighted_combine` (lsec_combine), and the pack / unpack-and-combine
// steps of `dcp_a2a_lse_reduce` (lsec_pack_send, lsec_unpack_combine,
// lsec_unpack); with the same kernels, the token-major merge of the page
// "vllm_ascend/attention/context_parallel/sfa_cp.py" (lsec_merge), the
// combine over strided receive planes of the direct exchange on the page
// "vllm.v1.attention.ops.dcp" (lsec_combine_planes), and the local step of
// the LSE all-gather strategies named there (lsec_correct_partial). The
// argument contract of each entry point is in lsec.h.
//
// Design. The combine is a streaming reduction: per (token, head) row it reads
// N planes of D values and writes one, so it is bound by HBM bandwidth at
// about one FMA per byte. It runs on plain VALU (no MFMA): a group of
// consecutive lanes owns a row, each lane moving one 16-byte chunk (8 bf16 /
// fp16 or 4 fp32 elements) per plane. The weights are computed in registers
// from the row's N LSE values and shared with 16-lane DPP reductions, so the
// combine keeps no data in LDS (its tiled launches reserve LDS only to cap
// occupancy). Packed rows are D + P elements wide (P = 2 for 16-bit elements,
// 1 for fp32), so a packed row starts only 4-byte aligned; gfx950 serves
// dwordx4 accesses at 4-byte alignment, so the receive side reads those rows
// in place, and the pack assembles its spans of rows in LDS to write them
// with aligned stores.
//
// Build with -Xclang -target-feature -Xclang -packed-fp32-ops and without
// fast-math (the NaN / infinity tests must survive).

#include <atomic>

#include "lsec_device.h"

namespace lsec_detail {
namespace {

// ---------------------------------------------------------------- combine (row kernel)
//
// For N = 1, N > 16, or D outside {128, 256, 512} (whole 16-byte chunks, at
// most 256 lanes per row). Row r of plane n starts at element n * plane + r * stride of `src`.
// Separate layout (lsec_combine): stride = D, plane >= rows * D (rows * D
// when dense; more when the planes are the leading rows of longer ones), LSE
// n of row r at lse[n * lse_plane + r]. Packed layout (lsec_unpack_combine):
// stride = D + P, plane = rows * (D + P), LSE = the fp32 in elements
// D .. D+P-1 of the row.
// Launch: a lane group of g = D / kEpc lanes owns a row; rows_per_block =
// kBlock / g. Every lane loads the row's N LSE values itself (broadcasts
// within the group) and issues all N chunk loads before it uses the first.
// SPLIT (an fp32 result from 16-bit partials): lane l owns elements
// [4l, 4l + 4) and [D/2 + 4l, D/2 + 4l + 4), read as two 8-byte loads, so each
// of its two 16-byte fp32 stores belongs to an instruction that writes one
// contiguous half of the row (D is a multiple of 8 here, so D/2 keeps every
// offset 8-byte aligned).
template <int DT, int NT, bool PACKED, bool SPLIT>
__global__ __launch_bounds__(kBlock) void combine_rows_kernel(
    const typename Elem<DT>::T* __restrict__ src, const float* __restrict__ lse, int n_rt,
    uint32_t rows, FastDiv g, uint32_t rows_per_block, int64_t stride, int64_t plane,
    int64_t lse_plane, int D, float scale, float inv_scale, void* __restrict__ out, int out_f32,
    float* __restrict__ out_lse, OutMap om) {
    constexpr int E = Elem<DT>::kEpc;
    const uint32_t t = threadIdx.x;
    const uint32_t rib = fdiv(t, g);
    const uint32_t lane = t - rib * g.d;
    if (rib >= rows_per_block) return;
    const uint32_t row = blockIdx.x * rows_per_block + rib;
    rows = valid_rows(rows, om);
    if (row >= rows) return;
    const int N = NT > 0 ? NT : n_rt;
    static_assert(!SPLIT || DT != LSEC_FP32, "fp32 partials already give fp32 results");
    const typename Elem<DT>::T* rp = src + int64_t(row) * stride;
    const typename Elem<DT>::T* cp = rp + lane * (SPLIT ? E / 2 : E);

    auto load_lse = [&](int n) -> float {
        if (PACKED) return ld_tail(rp + n * plane + D);
        return lse[int64_t(n) * lse_plane + row];
    };
    auto load_chunk = [&](int n) -> u32x4 {
        if constexpr (SPLIT) {
            const u32x2_a4 lo = __builtin_nontemporal_load(
                reinterpret_cast<const u32x2_a4*>(cp + n * plane));
            const u32x2_a4 hi = __builtin_nontemporal_load(
                reinterpret_cast<const u32x2_a4*>(cp + n * plane + D / 2));
            return u32x4{lo.x, lo.y, hi.x, hi.y};
        } else {
            if (PACKED) return ld16_a4(cp + n * plane);
            return ld16(cp + n * plane);
        }
    };

    float acc[E];
#pragma unroll
    for (int k = 0; k < E; ++k) acc[k] = kAccInit;
    float m, s;
    if constexpr (NT > 0) {
        float l[NT];
        u32x4 v[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) l[n] = load_lse(n);
#pragma unroll
        for (int n = 0; n < NT; ++n) v[n] = load_chunk(n);
        // Keep every load above this point: all N chunks stay in flight while
        // the weights are computed.
        __builtin_amdgcn_sched_barrier(0);
        m = -__builtin_inff();
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            l[n] = sanitize(l[n]);
            m = fmaxf(m, l[n]);
        }
        if (m == -__builtin_inff()) m = 0.0f;
        float w[NT];
        s = 0.0f;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            w[n] = weight(l[n] - m, scale);
            s += w[n];
        }
        const float inv = 1.0f / fmaxf(s, 1e-10f);
#pragma unroll
        for (int n = 0; n < NT; ++n) fma_chunk<DT>(v[n], w[n] * inv, acc);
    } else {
        m = -__builtin_inff();
        for (int n = 0; n < N; ++n) m = fmaxf(m, sanitize(load_lse(n)));
        if (m == -__builtin_inff()) m = 0.0f;
        s = 0.0f;
        for (int n = 0; n < N; ++n) s += weight(sanitize(load_lse(n)) - m, scale);
        const float inv = 1.0f / fmaxf(s, 1e-10f);
        for (int n0 = 0; n0 < N; n0 += 8) {
            u32x4 v[8];
            float w[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (n0 + k < N) {
                    v[k] = load_chunk(n0 + k);
                    w[k] = weight(sanitize(load_lse(n0 + k)) - m, scale) * inv;
                }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (n0 + k < N) fma_chunk<DT>(v[k], w[k], acc);
        }
    }
    const uint32_t orow = out_row(row, om);
    if constexpr (SPLIT) {
        float* p = static_cast<float*>(out) + uint64_t(orow) * D + lane * 4;
        st16(p, f32_chunk(acc[0], acc[1], acc[2], acc[3]));
        st16(p + D / 2, f32_chunk(acc[4], acc[5], acc[6], acc[7]));
    } else {
        store_chunk<DT>(out, uint64_t(orow) * D + lane * E, acc);
    }
    if (out_lse != nullptr && lane == 0) out_lse[orow] = global_lse(s, m, inv_scale);
}

// ---------------------------------------------------------------- combine (general path)
//
// Any D, element-aligned buffers. One thread per (row, element); each thread
// recomputes its row's weights. Packed rows read the LSE from its P tail
// elements (two 16-bit halves, or one fp32 element).
template <int DT, bool PACKED>
__global__ __launch_bounds__(kBlock) void combine_elems_kernel(
    const typename Elem<DT>::T* __restrict__ src, const float* __restrict__ lse, int N,
    int64_t rows, int64_t stride, int64_t plane, int64_t lse_plane, int64_t D, float scale,
    float inv_scale, void* __restrict__ out, int out_f32, float* __restrict__ out_lse,
    int64_t map_a, int64_t map_c, const int32_t* valid, int64_t rows_per_token) {
    if (valid != nullptr) {  // only the rows of the first *valid tokens
        const int32_t tv = *valid;
        const int64_t vr = tv <= 0 ? 0 : int64_t(tv) * rows_per_token;
        if (vr < rows) rows = vr;
    }
    const int64_t total = rows * D;
    for (int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x; i < total;
         i += int64_t(gridDim.x) * kBlock) {
        const int64_t row = i / D;
        const int64_t d = i - row * D;
        const typename Elem<DT>::T* rp = src + row * stride;
        auto load_lse = [&](int n) -> float {
            if (PACKED) {
                const typename Elem<DT>::T* q = rp + n * plane + D;
                if constexpr (Elem<DT>::kPack == 1)
                    return __uint_as_float(q[0]);
                else
                    return __uint_as_float(uint32_t(q[0]) | (uint32_t(q[1]) << 16));
            }
            return lse[int64_t(n) * lse_plane + row];
        };
        float m = -__builtin_inff();
        for (int n = 0; n < N; ++n) m = fmaxf(m, sanitize(load_lse(n)));
        if (m == -__builtin_inff()) m = 0.0f;
        float s = 0.0f;
        for (int n = 0; n < N; ++n) s += weight(sanitize(load_lse(n)) - m, scale);
        const float inv = 1.0f / fmaxf(s, 1e-10f);
        float acc = kAccInit;
        for (int n = 0; n < N; ++n) {
            float w = weight(sanitize(load_lse(n)) - m, scale) * inv;
            acc = fmaf(Elem<DT>::dec1(rp[n * plane + d]), w, acc);
        }
        const int64_t orow = map_a == 0 ? row : (row % map_c) * map_a + row / map_c;
        store_elem<DT>(out, orow * D + d, acc, out_f32);
        if (out_lse != nullptr && d == 0) out_lse[orow] = global_lse(s, m, inv_scale);
    }
}

// ---------------------------------------------------------------- correct a partial
//
// Local step of an LSE all-gather + output reduce-scatter (or all-reduce):
// with every shard's LSE gathered, rank r scales its own partial output by
// shard r's normalised weight; summing the scaled partials over the ranks
// gives the combine. Per row: the same sanitise / max / weight / clamped
// normalisation as the combine, then one plane read and one written.
// Tiled path for D in {128, 256, 512} and N <= 16: G = D / kEpc lanes per row,
// S row slots per lane, lane j of each 16-lane DPP row loads shard j's LSE.
// SPLIT (fp32 result from 16-bit partials) as in combine_tiled_kernel: a lane
// owns elements [4l, 4l + 4) and [D/2 + 4l, D/2 + 4l + 4) of its row.
template <int DT, int G, int S, bool SPLIT>
__global__ __launch_bounds__(kBlock) void correct_tiled_kernel(
    const float* __restrict__ lse, int N, int rank, const typename Elem<DT>::T* __restrict__ part,
    uint32_t rows, float scale, float inv_scale, void* __restrict__ out,
    float* __restrict__ out_lse) {
    static_assert(!SPLIT || DT != LSEC_FP32, "fp32 partials already give fp32 results");
    constexpr int E = Elem<DT>::kEpc;
    constexpr int RPS = kBlock / G;
    constexpr int D = G * E;
    const uint32_t t = threadIdx.x;
    const uint32_t rib = t / G;
    const uint32_t lane = t % G;
    const uint32_t j = t & 15u;
    const uint32_t row0 = xcd_chunked_block(blockIdx.x, gridDim.x) * (RPS * S);
    uint32_t row[S];
    float lw[S];
    u32x4 v[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        row[s] = row0 + s * RPS + rib;
        const uint32_t rc = row[s] < rows ? row[s] : rows - 1;
        lw[s] = int(j) < N ? lse[j * rows + rc] : -__builtin_inff();
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const uint32_t rc = row[s] < rows ? row[s] : rows - 1;
        if constexpr (SPLIT) {
            const auto* p = part + uint64_t(rc) * D + lane * (E / 2);
            const u32x2_a4 lo = __builtin_nontemporal_load(reinterpret_cast<const u32x2_a4*>(p));
            const u32x2_a4 hi = __builtin_nontemporal_load(reinterpret_cast<const u32x2_a4*>(p + D / 2));
            v[s] = u32x4{lo.x, lo.y, hi.x, hi.y};
        } else {
            v[s] = ld16(part + uint64_t(rc) * D + lane * E);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float l = int(j) < N ? sanitize(lw[s]) : -__builtin_inff();
        float m = row16_max(l);
        if (m == -__builtin_inff()) m = 0.0f;
        const float w = int(j) < N ? weight(l - m, scale) : 0.0f;
        const float sum = row16_sum(w);
        const float wr = lane_value<G>(w * (1.0f / fmaxf(sum, 1e-10f)), rank);
        if (row[s] < rows) {
            float acc[E];
#pragma unroll
            for (int k = 0; k < E; ++k) acc[k] = kAccInit;
            fma_chunk<DT>(v[s], wr, acc);
            if constexpr (SPLIT) {
                float* p = static_cast<float*>(out) + uint64_t(row[s]) * D + lane * 4;
                st16(p, f32_chunk(acc[0], acc[1], acc[2], acc[3]));
                st16(p + D / 2, f32_chunk(acc[4], acc[5], acc[6], acc[7]));
            } else {
                store_chunk<DT>(out, uint64_t(row[s]) * D + lane * E, acc);
            }
            if (out_lse != nullptr && lane == 0) out_lse[row[s]] = global_lse(sum, m, inv_scale);
        }
    }
}

// General path: any N, any D, element alignment; one thread per element.
template <int DT>
__global__ __launch_bounds__(kBlock) void correct_elems_kernel(
    const float* __restrict__ lse, int N, int rank, const typename Elem<DT>::T* __restrict__ part,
    int64_t rows, int64_t D, float scale, float inv_scale, void* __restrict__ out, int out_f32,
    float* __restrict__ out_lse) {
    const int64_t total = rows * D;
    for (int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x; i < total;
         i += int64_t(gridDim.x) * kBlock) {
        const int64_t row = i / D;
        const int64_t d = i - row * D;
        float m = -__builtin_inff();
        for (int n = 0; n < N; ++n) m = fmaxf(m, sanitize(lse[int64_t(n) * rows + row]));
        if (m == -__builtin_inff()) m = 0.0f;
        float s = 0.0f, wr = 0.0f;
        for (int n = 0; n < N; ++n) {
            const float w = weight(sanitize(lse[int64_t(n) * rows + row]) - m, scale);
            s += w;
            if (n == rank) wr = w;
        }
        wr *= 1.0f / fmaxf(s, 1e-10f);
        store_elem<DT>(out, i, fmaf(Elem<DT>::dec1(part[i]), wr, kAccInit), out_f32);
        if (out_lse != nullptr && d == 0) out_lse[row] = global_lse(s, m, inv_scale);
    }
}

// ---------------------------------------------------------------- pack (fast paths)
//
// Send row s = (r * B + b) * Hl + hl takes attention-output row
// src = b * H + r * Hl + hl: D elements, then the fp32 LSE's 32 bits in the P
// tail elements. T is the element word (2 or 4 bytes); the kernel moves bits
// only. A lane group of D / (16 / sizeof(T)) lanes owns a send row; each group
// handles kPackRows send rows (spaced one block-width apart) with all their
// loads in flight.
constexpr int kPackRows = 4;

template <typename T>
__global__ __launch_bounds__(kBlock) void pack_rows_kernel(
    const T* __restrict__ in, const float* __restrict__ lse, uint32_t send_rows, FastDiv g,
    uint32_t rows_per_block, FastDiv hl_div, FastDiv b_div, uint32_t H, int D,
    T* __restrict__ send) {
    constexpr int E = 16 / sizeof(T);
    constexpr int P = 4 / sizeof(T);
    const uint32_t t = threadIdx.x;
    const uint32_t rib = fdiv(t, g);
    const uint32_t lane = t - rib * g.d;
    if (rib >= rows_per_block) return;
    u32x4 v[kPackRows];
    float lv[kPackRows];
    uint32_t sr[kPackRows];
#pragma unroll
    for (int k = 0; k < kPackRows; ++k) {
        const uint32_t q = (blockIdx.x * kPackRows + k) * rows_per_block + rib;
        sr[k] = q;
        const uint32_t s = q < send_rows ? q : send_rows - 1;  // clamp: load a valid row, store nothing
        const uint32_t rb = fdiv(s, hl_div);
        const uint32_t hl = s - rb * hl_div.d;
        const uint32_t r = fdiv(rb, b_div);
        const uint32_t b = rb - r * b_div.d;
        const uint32_t src = b * H + r * hl_div.d + hl;
        v[k] = ld16(in + int64_t(src) * D + lane * E);
        lv[k] = lse[src];
    }
#pragma unroll
    for (int k = 0; k < kPackRows; ++k) {
        if (sr[k] < send_rows) {
            T* dp = send + int64_t(sr[k]) * (D + P);
            st16_a4(dp + lane * E, v[k]);
            if (lane == 0) st_tail(dp + D, lv[k]);
        }
    }
}

// Pack through LDS, persistent and pipelined (16-byte aligned send buffers).
// A tile is R = kPackRows * rows_per_block consecutive send rows: one
// contiguous span of R * (D + P) elements that starts on a 16-byte boundary,
// since R is a multiple of 4 and a packed row is 4 bytes past a multiple of
// 16. Its rows are assembled in LDS at their packed offsets (dword writes; the
// rows are only 4-byte aligned), and the span leaves as aligned, coalesced
// 16-byte non-temporal stores (8 % faster on MI355X than storing the 4-byte
// aligned rows directly, as pack_rows_kernel does). The grid holds
// kPackPipePerCu blocks per compute unit, block b walking tiles b,
// b + gridDim.x, ...; two LDS stages alternate: while tile i leaves its stage,
// the lanes already hold tile i + 1's loads, which then fill the other stage;
// one barrier per tile. The tile count of a block is uniform across it, so
// every barrier is reached by all its threads, and a block ends when its tiles
// run out (a launch whose blocks have one tile each reserves one stage).
// Measured on MI355X ([2048,64,128] bf16 -> 8 planes, cold): 2-3 % faster
// than one tile per block (1.07 x a plain copy of half its bytes against
// 1.10-1.11), 1 % for fp32; 2 or 4 blocks per CU, or a number that leaves the
// CUs uneven, measured slower than 3.
constexpr unsigned kPackPipePerCu = 3;

template <typename T>
__global__ __launch_bounds__(kBlock) void pack_pipe_kernel(
    const T* __restrict__ in, const float* __restrict__ lse, uint32_t send_rows, uint32_t tiles,
    FastDiv g, uint32_t rows_per_block, FastDiv hl_div, FastDiv b_div, uint32_t H, int D,
    T* __restrict__ send) {
    constexpr int E = 16 / sizeof(T);
    constexpr int P = 4 / sizeof(T);
    extern __shared__ __attribute__((aligned(16))) uint32_t stages[];
    const uint32_t t = threadIdx.x;
    const uint32_t rib = fdiv(t, g);
    const uint32_t lane = t - rib * g.d;
    const bool active = rib < rows_per_block;
    const uint32_t row_dw = uint32_t(D + P) * sizeof(T) / 4;  // dwords per packed row
    const uint32_t R = kPackRows * rows_per_block;
    const uint32_t stage_dw = R * row_dw;  // R is a multiple of 4: stage 1 is 16-byte aligned
    u32x4 v[kPackRows];
    float lv[kPackRows];
    auto load_tile = [&](uint32_t tile) {
        if (!active) return;
#pragma unroll
        for (int k = 0; k < kPackRows; ++k) {
            const uint32_t q = tile * R + k * rows_per_block + rib;
            const uint32_t s = q < send_rows ? q : send_rows - 1;  // clamp: load a valid row
            const uint32_t rb = fdiv(s, hl_div);
            const uint32_t hl = s - rb * hl_div.d;
            const uint32_t r = fdiv(rb, b_div);
            const uint32_t b = rb - r * b_div.d;
            const uint32_t src = b * H + r * hl_div.d + hl;
            v[k] = ld16(in + int64_t(src) * D + lane * E);
            lv[k] = lse[src];
        }
    };
    auto stage_tile = [&](uint32_t* stage) {
        if (!active) return;
#pragma unroll
        for (int k = 0; k < kPackRows; ++k) {
            uint32_t* rowp = stage + (k * rows_per_block + rib) * row_dw;
            uint32_t* cp = rowp + lane * 4;
            cp[0] = v[k].x;
            cp[1] = v[k].y;
            cp[2] = v[k].z;
            cp[3] = v[k].w;
            if (lane == 0) rowp[row_dw - 1] = __float_as_uint(lv[k]);  // the P tail elements
        }
    };
    auto store_tile = [&](uint32_t tile, const uint32_t* stage) {
        // Rows past send_rows were staged from clamped loads but are not stored.
        const uint32_t first = tile * R;
        const uint32_t nrows = send_rows - first < R ? send_rows - first : R;
        const uint32_t ndw = nrows * row_dw;
        uint32_t* dst = reinterpret_cast<uint32_t*>(send) + uint64_t(first) * row_dw;
        const uint32_t nfull = ndw / 4;
        for (uint32_t c = t; c < nfull; c += kBlock)
            __builtin_nontemporal_store(reinterpret_cast<const u32x4*>(stage)[c],
                                        reinterpret_cast<u32x4*>(dst) + c);
        for (uint32_t d = nfull * 4 + t; d < ndw; d += kBlock) dst[d] = stage[d];  // last tile's tail
    };
    uint32_t tile = blockIdx.x;
    if (tile >= tiles) return;  // uniform per block
    load_tile(tile);
    stage_tile(stages);
    __syncthreads();
    uint32_t cur = 0;
    for (;;) {
        const uint32_t next = tile + gridDim.x;
        const bool more = next < tiles;  // uniform per block
        if (more) load_tile(next);
        store_tile(tile, stages + cur * stage_dw);
        if (!more) break;
        stage_tile(stages + (cur ^ 1u) * stage_dw);
        __syncthreads();  // the next stage is whole, and the one just stored may be refilled
        tile = next;
        cur ^= 1u;
    }
}

// ---------------------------------------------------------------- pack (general path)
template <typename T>
__global__ __launch_bounds__(kBlock) void pack_elems_kernel(
    const T* __restrict__ in, const float* __restrict__ lse, int64_t B, int64_t H, int64_t Hl,
    int64_t D, int64_t total, T* __restrict__ send) {
    constexpr int P = 4 / sizeof(T);
    const int64_t W = D + P;
    for (int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x; i < total;
         i += int64_t(gridDim.x) * kBlock) {
        const int64_t s = i / W;
        const int64_t d = i - s * W;
        const int64_t rb = s / Hl;
        const int64_t hl = s - rb * Hl;
        const int64_t r = rb / B;
        const int64_t b = rb - r * B;
        const int64_t src = b * H + r * Hl + hl;
        T v;
        if (d < D) {
            v = in[src * D + d];
        } else {
            const uint32_t bits = __float_as_uint(lse[src]);
            if constexpr (P == 1)
                v = T(bits);
            else
                v = T(d == D ? (bits & 0xffffu) : (bits >> 16));
        }
        send[i] = v;
    }
}

// ---------------------------------------------------------------- unpack
template <typename T>
__global__ __launch_bounds__(kBlock) void unpack_rows_kernel(
    const T* __restrict__ recv, uint32_t total_rows, FastDiv g, uint32_t rows_per_block, int D,
    T* __restrict__ outs, float* __restrict__ lses) {
    constexpr int E = 16 / sizeof(T);
    constexpr int P = 4 / sizeof(T);
    const uint32_t t = threadIdx.x;
    const uint32_t rib = fdiv(t, g);
    const uint32_t lane = t - rib * g.d;
    if (rib >= rows_per_block) return;
    const uint32_t q = blockIdx.x * rows_per_block + rib;
    if (q >= total_rows) return;
    const T* sp = recv + int64_t(q) * (D + P);
    st16(outs + int64_t(q) * D + lane * E, ld16_a4(sp + lane * E));
    if (lane == 0) lses[q] = ld_tail(sp + D);
}

template <typename T>
__global__ __launch_bounds__(kBlock) void unpack_elems_kernel(
    const T* __restrict__ recv, int64_t total_rows, int64_t D, T* __restrict__ outs,
    float* __restrict__ lses) {
    constexpr int P = 4 / sizeof(T);
    const int64_t W = D + P;
    const int64_t total = total_rows * W;
    for (int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x; i < total;
         i += int64_t(gridDim.x) * kBlock) {
        const int64_t q = i / W;
        const int64_t d = i - q * W;
        if (d < D) {
            outs[q * D + d] = recv[i];
        } else if (d == D) {
            if constexpr (P == 1)
                lses[q] = __uint_as_float(uint32_t(recv[i]));
            else
                lses[q] = __uint_as_float(uint32_t(recv[i]) | (uint32_t(recv[i + 1]) << 16));
        }
    }
}

// ---------------------------------------------------------------- host side

constexpr float kLog2E = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }

unsigned general_grid(int64_t total) {
    int64_t blocks = (total + kBlock - 1) / kBlock;
    const int64_t cap = int64_t(1) << 20;  // grid-stride beyond this
    return unsigned(blocks < 1 ? 1 : (blocks > cap ? cap : blocks));
}

int launch_status() { return hipGetLastError() == hipSuccess ? LSEC_OK : LSEC_ERR_LAUNCH; }

// A `dtype` argument: the element type of the inputs, optionally with
// LSEC_OUT_FP32 (fp32 results from 16-bit inputs; fp32 inputs always give
// fp32 results). `esize` / `out_esize` are element sizes in bytes.
struct Dtype {
    int in;
    int out_f32;
    int64_t esize, out_esize;
};

bool parse_dtype(int code, bool allow_out_flag, Dtype* d) {
    const int in = code & ~LSEC_OUT_FP32;
    const bool flag = (code & LSEC_OUT_FP32) != 0;
    if (in != LSEC_BF16 && in != LSEC_FP16 && in != LSEC_FP32) return false;
    if (flag && !allow_out_flag) return false;
    d->in = in;
    d->out_f32 = (flag || in == LSEC_FP32) ? 1 : 0;
    d->esize = in == LSEC_FP32 ? 4 : 2;
    d->out_esize = d->out_f32 ? 4 : 2;
    return true;
}

// Fast kernels take D as whole 16-byte chunks, one lane each, within a block.
bool fast_d(int64_t D, int64_t esize) {
    const int64_t epc = 16 / esize;
    return D % epc == 0 && D / epc <= kBlock;
}

// Plane geometry of a combine: plane n of the partial outputs starts at
// element n * plane, its LSEs at n * lse_plane (separate layout).
struct Planes {
    int64_t plane, lse_plane;
};

template <int DT, int NT, bool PACKED>
void launch_combine_rows(const void* src, const float* lse, int N, uint32_t rows, int D,
                         Planes pl, float scale, float inv_scale, void* out, int out_f32,
                         float* out_lse, OutMap om, hipStream_t st) {
    const uint32_t g = uint32_t(D / Elem<DT>::kEpc);
    const uint32_t rpb = kBlock / g;
    const unsigned blocks = (rows + rpb - 1) / rpb;
    const int64_t stride = PACKED ? D + Elem<DT>::kPack : D;
    const auto* s = static_cast<const typename Elem<DT>::T*>(src);
    if constexpr (DT != LSEC_FP32) {
        if (out_f32) {
            launch(combine_rows_kernel<DT, NT, PACKED, true>, dim3(blocks), dim3(kBlock), 0, st,
                   s, lse, N, rows, make_fastdiv(g), rpb, stride, pl.plane, pl.lse_plane, D,
                   scale, inv_scale, out, out_f32, out_lse, om);
            return;
        }
    }
    launch(combine_rows_kernel<DT, NT, PACKED, false>, dim3(blocks), dim3(kBlock), 0, st, s, lse,
           N, rows, make_fastdiv(g), rpb, stride, pl.plane, pl.lse_plane, D, scale, inv_scale,
           out, out_f32, out_lse, om);
}

template <int DT, bool PACKED>
void dispatch_n(const void* src, const float* lse, int N, uint32_t rows, int D, Planes pl,
                float scale, float inv_scale, void* out, int out_f32, float* out_lse, OutMap om,
                hipStream_t st) {
#define LSEC_ROWS(NV) \
    launch_combine_rows<DT, NV, PACKED>(src, lse, N, rows, D, pl, scale, inv_scale, out, out_f32, out_lse, om, st)
    switch (N) {
        case 1: LSEC_ROWS(1); break;
        case 2: LSEC_ROWS(2); break;
        case 4: LSEC_ROWS(4); break;
        case 8: LSEC_ROWS(8); break;
        case 16: LSEC_ROWS(16); break;
        default: LSEC_ROWS(0); break;
    }
#undef LSEC_ROWS
}

// Tiled path: the largest S in {16, 8, 4, 2, 1} that still gives at least
// kTiledMinBlocks blocks (small inputs fall back to S = 1 with more planes in
// flight). With N = 16 a block walks enough planes to amortise its prologue
// (LSE loads, reductions) over 1024 blocks; with fewer planes it needs more,
// smaller blocks. Measured on MI355X (bf16): N=16 D=128 rows 2^19 -> S = 16;
// N=16 D=512 rows 2^16 -> S = 16; N=8 D=512 rows 2^16 -> S = 8;
// N=8 D=256 rows 2^17 -> S = 8; N=8 D=128 rows 2^17 -> S = 4.
constexpr uint64_t kTiledMinBlocks = 2048;
constexpr uint64_t kTiledMinBlocksN16 = 1024;

// Which combine kernel serves a call. `fast` = fast_d(D), rows < 2^31 and the
// buffers meet the 16-byte (separate) or 4-byte (packed) alignment; otherwise
// the element-wise kernel runs.
enum { kPathTiled = 0, kPathRows = 1, kPathElems = 2, kPathSpan = 3 };
struct CombinePlan {
    int kind;
    int S;  // row slots per lane (tiled path)
};

// `pl` gives the plane geometry of the separate layout (packed planes are
// always dense). `span_ok`: packed rows, a result in the input dtype, planes
// 16-byte aligned, identity output order and no valid count -- then the calls
// that would run the tiled kernel with S = 1 on rows of 128 values with N = 2,
// 4, 8 or 16 run a span kernel when the rows are a multiple of 4
// (combine_span_kernel for 16-bit elements, combine_span32_kernel for fp32).
CombinePlan plan_combine(int64_t N, int64_t rows, int64_t D, int64_t esize, bool packed,
                         bool fast, Planes pl, bool span_ok = false) {
    if (!fast) return {kPathElems, 0};
    const bool tiled_shape = (D == 128 || D == 256 || D == 512) && N >= 2 && N <= 16;
    if (tiled_shape) {
        const int64_t P = 4 / esize;
        const uint64_t plane_bytes =
            packed ? uint64_t(rows) * uint64_t(D + P) * uint64_t(esize) : uint64_t(pl.plane) * uint64_t(esize);
        const bool fits32 = plane_bytes < (uint64_t(1) << 32) &&
                            (packed || uint64_t(N) * uint64_t(pl.lse_plane) < (uint64_t(1) << 32));
        if (fits32) {
            const uint64_t rps = kBlock / uint64_t(D * esize / 16);
            const uint64_t min_blocks = N >= 16 ? kTiledMinBlocksN16 : kTiledMinBlocks;
            int S = 16;
            while (S > 1 && (uint64_t(rows) + rps * S - 1) / (rps * S) < min_blocks) S /= 2;
            if (S == 1 && span_ok && packed && (esize == 2 || esize == 4) && D == 128 &&
                rows % 4 == 0 &&
                (N == 2 || N == 4 || N == 8 || N == 16))
                return {kPathSpan, 1};
            return {kPathTiled, S};
        }
    }
    return {kPathRows, 0};
}

template <int DT, bool PACKED>
void run_combine_dt(const void* src, const float* lse, int64_t N, int64_t rows, int64_t D,
                    Planes pl, float scale, float inv_scale, void* out, int out_f32,
                    float* out_lse, const CombinePlan& plan, OutMap om, int64_t map_a,
                    int64_t map_c, hipStream_t st) {
    if (plan.kind == kPathTiled || plan.kind == kPathSpan) {
        const int64_t stride = PACKED ? D + Elem<DT>::kPack : D;
        const TiledArgs a{src, lse, int(N), uint32_t(rows), uint32_t(stride),
                          uint64_t(pl.plane) * sizeof(typename Elem<DT>::T), uint32_t(pl.lse_plane),
                          scale, inv_scale, out, out_f32, out_lse, om, st};
        if constexpr (PACKED) {
            if (plan.kind == kPathSpan) {
                launch_span<DT>(int(N), a);
                return;
            }
        }
        launch_tiled<DT, PACKED>(int(N), plan.S, int(D), a);
    } else if (plan.kind == kPathRows) {
        dispatch_n<DT, PACKED>(src, lse, int(N), uint32_t(rows), int(D), pl, scale, inv_scale,
                               out, out_f32, out_lse, om, st);
    } else {
        const int64_t stride = PACKED ? D + Elem<DT>::kPack : D;
        launch(combine_elems_kernel<DT, PACKED>, dim3(general_grid(rows * D)), dim3(kBlock), 0,
               st, static_cast<const typename Elem<DT>::T*>(src), lse, int(N), rows, stride,
               pl.plane, pl.lse_plane, D, scale, inv_scale, out, out_f32, out_lse, map_a, map_c,
               om.valid, int64_t(om.rows_per_token));
    }
}

// Runs a validated combine. `pl` is the plane geometry in elements; packed
// planes are dense (plane = rows * (D + P); lse_plane unused).
template <bool PACKED>
int run_combine(const void* src, const float* lse, int64_t N, int64_t rows, int64_t D,
                const Dtype& dt, int base, void* out, float* out_lse, bool fast, hipStream_t st,
                Planes pl, int64_t map_a = 0, int64_t map_c = 1, const int32_t* valid = nullptr,
                int64_t rows_per_token = 0) {
    const OutMap om{uint32_t(map_a), make_fastdiv(uint32_t(map_c)), valid,
                    uint32_t(rows_per_token)};
    const float scale = base == LSEC_BASE_2 ? 1.0f : kLog2E;
    const float inv_scale = base == LSEC_BASE_2 ? 1.0f : kLn2;
    const bool span_ok = PACKED && dt.out_esize == dt.esize && aligned(src, 16) && map_a == 0 &&
                         valid == nullptr;
    const CombinePlan plan = plan_combine(N, rows, D, dt.esize, PACKED, fast, pl, span_ok);
    (void)hipGetLastError();
#define LSEC_RUN(DTV)                                                                        \
    run_combine_dt<DTV, PACKED>(src, lse, N, rows, D, pl, scale, inv_scale, out, dt.out_f32, \
                                out_lse, plan, om, map_a, map_c, st)
    switch (dt.in) {
        case LSEC_BF16: LSEC_RUN(LSEC_BF16); break;
        case LSEC_FP16: LSEC_RUN(LSEC_FP16); break;
        default: LSEC_RUN(LSEC_FP32); break;
    }
#undef LSEC_RUN
    return launch_status();
}

template <int DT, int G, bool SPLIT>
void launch_correct_s(int S, const float* lse, int N, int rank, const void* part, uint32_t rows,
                      float scale, float inv_scale, void* out, float* out_lse, hipStream_t st) {
    constexpr uint32_t RPS = kBlock / G;
    const unsigned blocks = (rows + RPS * S - 1) / (RPS * S);
    const auto* p = static_cast<const typename Elem<DT>::T*>(part);
#define LSEC_CORRECT(SV)                                                                     \
    launch(correct_tiled_kernel<DT, G, SV, SPLIT>, dim3(blocks), dim3(kBlock), 0, st, lse, N, \
           rank, p, rows, scale, inv_scale, out, out_lse)
    switch (S) {
        case 8: LSEC_CORRECT(8); break;
        case 4: LSEC_CORRECT(4); break;
        case 2: LSEC_CORRECT(2); break;
        default: LSEC_CORRECT(1); break;
    }
#undef LSEC_CORRECT
}

template <int DT>
void launch_correct(bool tiled, const float* lse, int64_t N, int64_t rank, const void* part,
                    int64_t rows, int64_t D, float scale, float inv_scale, void* out,
                    int out_f32, float* out_lse, hipStream_t st) {
    if (!tiled) {
        launch(correct_elems_kernel<DT>, dim3(general_grid(rows * D)), dim3(kBlock), 0, st, lse,
               int(N), int(rank), static_cast<const typename Elem<DT>::T*>(part), rows, D, scale,
               inv_scale, out, out_f32, out_lse);
        return;
    }
    constexpr int E = Elem<DT>::kEpc;
    const uint64_t rps = kBlock / uint64_t(D / E);
    int S = 8;
    while (S > 1 && (uint64_t(rows) + rps * S - 1) / (rps * S) < kTiledMinBlocks) S /= 2;
#define LSEC_CORRECT_G(GV, SPLIT) \
    launch_correct_s<DT, GV, SPLIT>(S, lse, int(N), int(rank), part, uint32_t(rows), scale, inv_scale, out, out_lse, st)
    constexpr bool kCanSplit = DT != LSEC_FP32;
    if (kCanSplit && out_f32) {
        switch (D) {
            case 128: LSEC_CORRECT_G(128 / E, kCanSplit); break;
            case 256: LSEC_CORRECT_G(256 / E, kCanSplit); break;
            default: LSEC_CORRECT_G(512 / E, kCanSplit); break;
        }
    } else {
        switch (D) {
            case 128: LSEC_CORRECT_G(128 / E, false); break;
            case 256: LSEC_CORRECT_G(256 / E, false); break;
            default: LSEC_CORRECT_G(512 / E, false); break;
        }
    }
#undef LSEC_CORRECT_G
}

// Which pack kernel serves a call. `in_aligned`: attn_out is 16-byte aligned;
// `send_align`: the send buffer's alignment in bytes (16, 4 or the element
// size). Whole 16-byte chunks per lane need fast_d(D), rows < 2^31, an aligned
// input and a 4-byte aligned send buffer; with a 16-byte aligned one the rows
// go out through LDS in whole cache lines, by a persistent grid that overlaps
// each tile's stores with the next tile's loads.
enum { kPackPathElems = 0, kPackPathRows = 1, kPackPathPipe = 2 };

int plan_pack(int64_t D, int64_t esize, int64_t rows, bool in_aligned, int send_align) {
    if (!(fast_d(D, esize) && rows < (int64_t(1) << 31) && in_aligned && send_align >= 4))
        return kPackPathElems;
    return send_align < 16 ? kPackPathRows : kPackPathPipe;
}

int send_alignment(const void* p, int64_t esize) {
    return aligned(p, 16) ? 16 : (aligned(p, 4) ? 4 : int(esize));
}

// Compute units of the device `st` runs on (256 on MI355X), queried once per
// device. Only the pipelined pack's grid depends on it; a failed query counts
// 256.
unsigned cu_count(hipStream_t st) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = -1;
    if (hipStreamGetDevice(st, &dev) != hipSuccess && hipGetDevice(&dev) != hipSuccess) dev = -1;
    if (dev < 0 || dev >= kMaxDevices) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return unsigned(n);
}

template <typename T>
void launch_pack(int kind, const void* attn_out, const float* lse, int64_t B, int64_t H,
                 int64_t Hl, int64_t D, int64_t rows, int64_t total, unsigned cus, void* send,
                 hipStream_t st) {
    const T* in = static_cast<const T*>(attn_out);
    T* dst = static_cast<T*>(send);
    if (kind == kPackPathElems) {
        launch(pack_elems_kernel<T>, dim3(general_grid(total)), dim3(kBlock), 0, st, in, lse, B,
               H, Hl, D, total, dst);
        return;
    }
    const uint32_t g = uint32_t(D / (16 / sizeof(T)));
    const uint32_t rpb = kBlock / g;
    const uint32_t R = kPackRows * rpb;  // send rows per tile
    const uint32_t tiles = uint32_t((rows + R - 1) / R);
    if (kind == kPackPathRows) {
        launch(pack_rows_kernel<T>, dim3(tiles), dim3(kBlock), 0, st, in, lse, uint32_t(rows),
               make_fastdiv(g), rpb, make_fastdiv(uint32_t(Hl)), make_fastdiv(uint32_t(B)),
               uint32_t(H), int(D), dst);
        return;
    }
    const unsigned grid = kPackPipePerCu * cus;
    const unsigned blocks = tiles < grid ? tiles : grid;
    const size_t stage_bytes = size_t(R) * size_t(D + 4 / sizeof(T)) * sizeof(T);
    launch(pack_pipe_kernel<T>, dim3(blocks), dim3(kBlock), (tiles > blocks ? 2 : 1) * stage_bytes,
           st, in, lse, uint32_t(rows), tiles, make_fastdiv(g), rpb, make_fastdiv(uint32_t(Hl)),
           make_fastdiv(uint32_t(B)), uint32_t(H), int(D), dst);
}

template <typename T>
void launch_unpack(bool fast, const void* recv, int64_t total_rows, int64_t D, int64_t total,
                   void* outputs, float* lses, hipStream_t st) {
    const T* src = static_cast<const T*>(recv);
    T* outs = static_cast<T*>(outputs);
    if (fast) {
        const uint32_t g = uint32_t(D / (16 / sizeof(T)));
        const uint32_t rpb = kBlock / g;
        const unsigned blocks = unsigned((total_rows + rpb - 1) / rpb);
        launch(unpack_rows_kernel<T>, dim3(blocks), dim3(kBlock), 0, st, src, uint32_t(total_rows),
               make_fastdiv(g), rpb, int(D), outs, lses);
    } else {
        launch(unpack_elems_kernel<T>, dim3(general_grid(total)), dim3(kBlock), 0, st, src,
               total_rows, D, outs, lses);
    }
}

// Shared by lsec_combine, lsec_merge and lsec_combine_planes(_valid): rows
// (b, h) of a [B, H] grid, stored in input order or, when `transposed`, at row
// h * B + b. Plane n of the partial outputs starts at element n * plane_stride,
// its LSEs at n * lse_plane_stride; the first B * H rows of each plane are
// combined, or, when `masked`, those of the first query_start_loc[num_reqs]
// tokens b (read by the kernels).
int combine_entry(const void* outputs, int64_t plane_stride, const float* lses,
                  int64_t lse_plane_stride, int64_t N, int64_t B, int64_t H, int64_t D, int dtype,
                  int base, void* out, float* out_lse, void* stream, bool transposed,
                  bool masked = false, const int32_t* query_start_loc = nullptr,
                  int64_t num_reqs = 0) {
    if (N < 1 || B < 0 || H < 1 || D < 1 || N > (int64_t(1) << 30)) return LSEC_ERR_SHAPE;
    Dtype dt;
    if (!parse_dtype(dtype, true, &dt)) return LSEC_ERR_DTYPE;
    if (base != LSEC_BASE_E && base != LSEC_BASE_2) return LSEC_ERR_BASE;
    int64_t rows, rd, ob, span, lspan;
    if (!mul_ok(B, H, &rows) || !mul_ok(rows, D, &rd) || !mul_ok(rd, dt.out_esize, &ob))
        return LSEC_ERR_SHAPE;
    if (plane_stride < rd || lse_plane_stride < rows || num_reqs < 0 ||
        (masked && H > int64_t(UINT32_MAX)))
        return LSEC_ERR_SHAPE;
    if (!mul_ok(N - 1, plane_stride, &span) || __builtin_add_overflow(span, rd, &span) ||
        !mul_ok(span, dt.esize, &span) || !mul_ok(N - 1, lse_plane_stride, &lspan) ||
        __builtin_add_overflow(lspan, rows, &lspan) || !mul_ok(lspan, 4, &lspan))
        return LSEC_ERR_SHAPE;
    if (rows == 0) return LSEC_OK;
    if (!outputs || !lses || !out || (masked && !query_start_loc)) return LSEC_ERR_NULL;
    if (!aligned(outputs, dt.esize) || !aligned(out, dt.out_esize) || !aligned(lses, 4) ||
        (out_lse && !aligned(out_lse, 4)) || (masked && !aligned(query_start_loc, 4)))
        return LSEC_ERR_ALIGNMENT;
    const bool fast = fast_d(D, dt.esize) && rows < (int64_t(1) << 31) && aligned(outputs, 16) &&
                      aligned(out, 16) && (plane_stride * dt.esize) % 16 == 0;
    return run_combine<false>(outputs, lses, N, rows, D, dt, base, out, out_lse, fast,
                              static_cast<hipStream_t>(stream), Planes{plane_stride, lse_plane_stride},
                              transposed ? B : 0, transposed ? H : 1,
                              masked ? query_start_loc + num_reqs : nullptr, H);
}

}  // namespace
}  // namespace lsec_detail

using namespace lsec_detail;

// ---------------------------------------------------------------- C ABI

extern "C" {

int lsec_version(void) { return 200; }

int lsec_pack_dim(int dtype) {
    if (dtype == LSEC_BF16 || dtype == LSEC_FP16) return 2;
    return dtype == LSEC_FP32 ? 1 : -1;
}

const char* lsec_status_string(int status) {
    switch (status) {
        case LSEC_OK: return "ok";
        case LSEC_ERR_NULL: return "a required pointer is NULL";
        case LSEC_ERR_SHAPE: return "invalid shape (need N >= 1, B >= 0, H >= 1, D >= 1, sizes within int64)";
        case LSEC_ERR_DIVISIBILITY: return "H must be divisible by N";
        case LSEC_ERR_DTYPE:
            return "unsupported dtype (bf16, fp16 or fp32; LSEC_OUT_FP32 only on combining calls)";
        case LSEC_ERR_ALIGNMENT: return "a pointer is not aligned to its element size";
        case LSEC_ERR_BASE: return "base must be LSEC_BASE_E or LSEC_BASE_2";
        case LSEC_ERR_LAUNCH: return "kernel launch failed";
        case LSEC_ERR_TOKEN_DIM: return "token_dim must be 1 or 2";
        case LSEC_ERR_RANK: return "rank must be in [0, N)";
        default: return "unknown status";
    }
}

const char* lsec_pack_path(int64_t N, int64_t B, int64_t H, int64_t D, int dtype, int in_aligned,
                           int send_align) {
    Dtype dt;
    if (N < 1 || B < 1 || H < 1 || D < 1 || H % N != 0 || !parse_dtype(dtype, false, &dt))
        return "none";
    int64_t rows;
    if (!mul_ok(B, H, &rows)) return "none";
    const int sa = send_align >= 16 ? 16 : (send_align >= 4 ? 4 : int(dt.esize));
    switch (plan_pack(D, dt.esize, rows, in_aligned != 0, sa)) {
        case kPackPathPipe: return "pack_pipe_kernel";
        case kPackPathRows: return "pack_rows_kernel";
        default: return "pack_elems_kernel";
    }
}

const char* lsec_combine_path(int64_t N, int64_t B, int64_t H, int64_t D, int dtype, int packed,
                              int aligned_buffers) {
    int64_t rows;
    Dtype dt;
    if (N < 1 || B < 1 || H < 1 || D < 1 || !mul_ok(B, H, &rows) || !parse_dtype(dtype, true, &dt))
        return "none";
    const bool fast = aligned_buffers && fast_d(D, dt.esize) && rows < (int64_t(1) << 31);
    int64_t rd;
    if (!mul_ok(rows, D, &rd)) return "none";
    const bool span_ok = packed && aligned_buffers && dt.out_esize == dt.esize;
    const CombinePlan plan =
        plan_combine(N, rows, D, dt.esize, packed != 0, fast, Planes{rd, rows}, span_ok);
    if (plan.kind == kPathElems) return "combine_elems_kernel";
    if (plan.kind == kPathSpan) return dt.esize == 2 ? "combine_span_kernel" : "combine_span32_kernel";
    if (plan.kind == kPathRows) return "combine_rows_kernel";
    switch (plan.S) {
        case 16: return "combine_tiled_kernel S=16";
        case 8: return "combine_tiled_kernel S=8";
        case 4: return "combine_tiled_kernel S=4";
        case 2: return "combine_tiled_kernel S=2";
        default: return "combine_tiled_kernel S=1";
    }
}

// Dense planes: plane stride B*H*D elements, LSE plane stride B*H. When
// those products overflow, combine_entry rejects the call (SHAPE).
static int64_t dense_or_max(int64_t a, int64_t b, int64_t c) {
    int64_t r;
    if (a < 0 || b < 0 || c < 0 || !mul_ok(a, b, &r) || !mul_ok(r, c, &r)) return INT64_MAX;
    return r;
}

int lsec_combine(const void* outputs, const float* lses, int64_t N, int64_t B, int64_t H,
                 int64_t D, int dtype, int base, void* out, float* out_lse, void* stream) {
    return combine_entry(outputs, dense_or_max(B, H, D), lses, dense_or_max(B, H, 1), N, B, H, D,
                         dtype, base, out, out_lse, stream, false);
}

int lsec_combine_planes(const void* outputs, int64_t plane_stride, const float* lses,
                        int64_t lse_plane_stride, int64_t N, int64_t T, int64_t H, int64_t D,
                        int dtype, int base, void* out, float* out_lse, void* stream) {
    return combine_entry(outputs, plane_stride, lses, lse_plane_stride, N, T, H, D, dtype, base,
                         out, out_lse, stream, false);
}

int lsec_combine_planes_valid(const void* outputs, int64_t plane_stride, const float* lses,
                              int64_t lse_plane_stride, int64_t N, int64_t T, int64_t H,
                              int64_t D, int dtype, int base, const int32_t* query_start_loc,
                              int64_t num_reqs, void* out, float* out_lse, void* stream) {
    return combine_entry(outputs, plane_stride, lses, lse_plane_stride, N, T, H, D, dtype, base,
                         out, out_lse, stream, false, true, query_start_loc, num_reqs);
}

int lsec_merge(const void* outputs, const float* lses, int64_t N, int64_t A, int64_t C,
               int64_t D, int token_dim, int dtype, int base, void* out, float* out_lse,
               void* stream) {
    if (token_dim != 1 && token_dim != 2) return LSEC_ERR_TOKEN_DIM;
    return combine_entry(outputs, dense_or_max(A, C, D), lses, dense_or_max(A, C, 1), N, A, C, D,
                         dtype, base, out, out_lse, stream, token_dim == 2);
}

int lsec_unpack_combine(const void* recv, int64_t N, int64_t B, int64_t Hl, int64_t D, int dtype,
                        int base, void* out, float* out_lse, void* stream) {
    if (N < 1 || B < 0 || Hl < 1 || D < 1 || N > (int64_t(1) << 30)) return LSEC_ERR_SHAPE;
    Dtype dt;
    if (!parse_dtype(dtype, true, &dt)) return LSEC_ERR_DTYPE;
    if (base != LSEC_BASE_E && base != LSEC_BASE_2) return LSEC_ERR_BASE;
    const int64_t P = 4 / dt.esize;
    int64_t rows, rw, all, rd;
    if (!mul_ok(B, Hl, &rows) || !mul_ok(rows, D + P, &rw) || !mul_ok(rw, N, &all) ||
        !mul_ok(all, dt.esize, &all) || !mul_ok(rows, D, &rd) || !mul_ok(rd, dt.out_esize, &rd))
        return LSEC_ERR_SHAPE;
    if (rows == 0) return LSEC_OK;
    if (!recv || !out) return LSEC_ERR_NULL;
    if (!aligned(recv, dt.esize) || !aligned(out, dt.out_esize) || (out_lse && !aligned(out_lse, 4)))
        return LSEC_ERR_ALIGNMENT;
    const bool fast = fast_d(D, dt.esize) && rows < (int64_t(1) << 31) && aligned(recv, 4) &&
                      aligned(out, 16);
    return run_combine<true>(recv, nullptr, N, rows, D, dt, base, out, out_lse, fast,
                             static_cast<hipStream_t>(stream), Planes{rows * (D + P), 0});
}

int lsec_correct_partial(const float* lses, int64_t N, int64_t rank, const void* partial,
                         int64_t B, int64_t H, int64_t D, int dtype, int base, void* out,
                         float* out_lse, void* stream) {
    if (N < 1 || B < 0 || H < 1 || D < 1 || N > (int64_t(1) << 30)) return LSEC_ERR_SHAPE;
    if (rank < 0 || rank >= N) return LSEC_ERR_RANK;
    Dtype dt;
    if (!parse_dtype(dtype, true, &dt)) return LSEC_ERR_DTYPE;
    if (base != LSEC_BASE_E && base != LSEC_BASE_2) return LSEC_ERR_BASE;
    int64_t rows, rd, ib, ob, nl;
    if (!mul_ok(B, H, &rows) || !mul_ok(rows, D, &rd) || !mul_ok(rd, dt.esize, &ib) ||
        !mul_ok(rd, dt.out_esize, &ob) || !mul_ok(rows, N, &nl) || !mul_ok(nl, 4, &nl))
        return LSEC_ERR_SHAPE;
    if (rows == 0) return LSEC_OK;
    if (!lses || !partial || !out) return LSEC_ERR_NULL;
    if (!aligned(partial, dt.esize) || !aligned(out, dt.out_esize) || !aligned(lses, 4) ||
        (out_lse && !aligned(out_lse, 4)))
        return LSEC_ERR_ALIGNMENT;
    const bool tiled = (D == 128 || D == 256 || D == 512) && N <= 16 &&
                       rows < (int64_t(1) << 31) && uint64_t(N) * uint64_t(rows) < (uint64_t(1) << 32) &&
                       aligned(partial, 16) && aligned(out, 16);
    const float scale = base == LSEC_BASE_2 ? 1.0f : kLog2E;
    const float inv_scale = base == LSEC_BASE_2 ? 1.0f : kLn2;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
#define LSEC_CORRECT_DT(DTV) \
    launch_correct<DTV>(tiled, lses, N, rank, partial, rows, D, scale, inv_scale, out, dt.out_f32, out_lse, st)
    switch (dt.in) {
        case LSEC_BF16: LSEC_CORRECT_DT(LSEC_BF16); break;
        case LSEC_FP16: LSEC_CORRECT_DT(LSEC_FP16); break;
        default: LSEC_CORRECT_DT(LSEC_FP32); break;
    }
#undef LSEC_CORRECT_DT
    return launch_status();
}

int lsec_pack_send(const void* attn_out, const float* attn_lse, int64_t N, int64_t B, int64_t H,
                   int64_t D, int dtype, void* send, void* stream) {
    if (N < 1 || B < 0 || H < 1 || D < 1) return LSEC_ERR_SHAPE;
    if (H % N != 0) return LSEC_ERR_DIVISIBILITY;
    Dtype dt;
    if (!parse_dtype(dtype, false, &dt)) return LSEC_ERR_DTYPE;
    const int64_t P = 4 / dt.esize;
    int64_t rows, total, bytes;
    if (!mul_ok(B, H, &rows) || !mul_ok(rows, D + P, &total) || !mul_ok(total, dt.esize, &bytes))
        return LSEC_ERR_SHAPE;
    if (rows == 0) return LSEC_OK;
    if (!attn_out || !attn_lse || !send) return LSEC_ERR_NULL;
    if (!aligned(attn_out, dt.esize) || !aligned(send, dt.esize) || !aligned(attn_lse, 4))
        return LSEC_ERR_ALIGNMENT;
    const int64_t Hl = H / N;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int kind =
        plan_pack(D, dt.esize, rows, aligned(attn_out, 16), send_alignment(send, dt.esize));
    const unsigned cus = kind == kPackPathPipe ? cu_count(st) : 0;
    (void)hipGetLastError();
    if (dt.esize == 4)
        launch_pack<uint32_t>(kind, attn_out, attn_lse, B, H, Hl, D, rows, total, cus, send, st);
    else
        launch_pack<uint16_t>(kind, attn_out, attn_lse, B, H, Hl, D, rows, total, cus, send, st);
    return launch_status();
}

int lsec_unpack(const void* recv, int64_t N, int64_t B, int64_t Hl, int64_t D, int dtype,
                void* outputs, float* lses, void* stream) {
    if (N < 1 || B < 0 || Hl < 1 || D < 1) return LSEC_ERR_SHAPE;
    Dtype dt;
    if (!parse_dtype(dtype, false, &dt)) return LSEC_ERR_DTYPE;
    const int64_t P = 4 / dt.esize;
    int64_t rows, total_rows, total, bytes;
    if (!mul_ok(B, Hl, &rows) || !mul_ok(rows, N, &total_rows) ||
        !mul_ok(total_rows, D + P, &total) || !mul_ok(total, dt.esize, &bytes))
        return LSEC_ERR_SHAPE;
    if (total_rows == 0) return LSEC_OK;
    if (!recv || !outputs || !lses) return LSEC_ERR_NULL;
    if (!aligned(recv, dt.esize) || !aligned(outputs, dt.esize) || !aligned(lses, 4))
        return LSEC_ERR_ALIGNMENT;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const bool fast = fast_d(D, dt.esize) && total_rows < (int64_t(1) << 31) && aligned(recv, 4) &&
                      aligned(outputs, 16);
    if (dt.esize == 4)
        launch_unpack<uint32_t>(fast, recv, total_rows, D, total, outputs, lses, st);
    else
        launch_unpack<uint16_t>(fast, recv, total_rows, D, total, outputs, lses, st);
    return launch_status();
}

}  // extern "C"
