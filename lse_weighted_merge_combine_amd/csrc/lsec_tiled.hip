// lsec_tiled.hip -- the tiled combine of liblsec.so for one element type,
// compiled once per type (LSEC_TILED_DT = LSEC_BF16, LSEC_FP16, LSEC_FP32) so
// that its many instantiations build in parallel. The host code in lsec.hip
// calls launch_tiled<DT, PACKED> and, for packed rows of 128 16-bit values,
// launch_span<DT>, instantiated at the end of this file.
//
// Build with -Xclang -target-feature -Xclang -packed-fp32-ops and without
// fast-math (the NaN / infinity tests must survive).

#include "lsec_device.h"

#ifndef LSEC_TILED_DT
#error "compile with -DLSEC_TILED_DT=<LSEC_BF16 | LSEC_FP16 | LSEC_FP32>"
#endif

namespace lsec_detail {
namespace {

// ---------------------------------------------------------------- combine (tiled path)
//
// For D in {128, 256, 512} and 2 <= N <= 16 (N = 2, 4, 8, 16 compiled in; other
// N at run time, NT = 0, with the plane groups of N = 16 and the planes past N
// skipped by a uniform branch). A row is owned by
// G = D / kEpc lanes (16 bytes each). A block of 256 threads covers S slots of
// 256/G consecutive rows, so per plane it reads one contiguous run of
// S*256/G rows (32 KB at S = 8). The planes are walked in order, PG at a time:
// each lane has PG*S 16-byte loads in flight and a block keeps few DRAM pages
// open. On MI355X this streams markedly faster than issuing all N planes of
// one row at once, which spreads every block over N distant pages.
//
// Weights: lane j of each 16-lane DPP row loads shard j's LSE for its row
// (j < N; the 16-lane segments of a row group hold identical copies). Max and
// sum are 16-lane DPP reductions; during the sweep the weight of plane n comes
// from lane n of the segment (a lane shuffle, or readlane when a wave holds
// one row or part of one). The global LSE is written before the sweep so
// nothing but the weights stays live through it.
//
// Addresses: plane n starts at n * plane_bytes (uniform, scalar registers);
// a lane's chunk sits at a 32-bit byte offset inside the plane; shard j's LSE
// of row r is lse[j * lse_plane + r]. The host checks plane_bytes < 2^32 and
// N * lse_plane < 2^32. Rows past the end of the last block are clamped to
// the last row for loading and are not stored.
__device__ __forceinline__ u32x4 ld16_nt_at(const char* p) { return ld16(p); }
__device__ __forceinline__ u32x4 ld16_a4_at(const char* p) { return ld16_a4(p); }

template <int S, int NT>
constexpr int tiled_pg() {
    return (S >= 4 ? 1 : (8 / S < NT ? 8 / S : NT));
}

// SPLIT (fp32 result from 16-bit partials): lane l of a row owns elements
// [4l, 4l + 4) and [D/2 + 4l, D/2 + 4l + 4) instead of [8l, 8l + 8), read as
// two 8-byte loads, so each of its two 16-byte fp32 stores belongs to an
// instruction that writes one contiguous half of the row (whole cache
// lines). Measured on MI355X: 6.6 % faster on N=16 D=128 2^19 rows, 4.5 % on
// N=8 D=512 2^16 rows, than 16-byte loads with two interleaved stores.
// Otherwise the result has the input dtype.
template <int DT, int NT, int G, int S, bool PACKED, bool SPLIT>
__global__ __launch_bounds__(kBlock) void combine_tiled_kernel(
    const void* src, const float* __restrict__ lse, int n_rt, uint32_t rows, uint32_t stride,
    uint64_t plane_bytes, uint32_t lse_plane, float scale, float inv_scale,
    void* __restrict__ out, float* __restrict__ out_lse, OutMap om) {
    static_assert(!SPLIT || DT != LSEC_FP32, "fp32 partials already give fp32 results");
    constexpr int E = Elem<DT>::kEpc;
    constexpr uint32_t ES = sizeof(typename Elem<DT>::T);
    constexpr int RPS = kBlock / G;  // rows per slot
    constexpr int D = G * E;
    constexpr int PG = tiled_pg<S, (NT > 0 ? NT : 16)>();
    static_assert(NT == 0 || NT % PG == 0, "plane groups must tile N");
    const int N = NT > 0 ? NT : n_rt;  // 2 <= n_rt <= 16
    // Plane n0 + p exists (always for a compiled-in N).
    auto has = [&](int n) { return NT > 0 || n < N; };
    static_assert(RPS >= 1 && kBlock % G == 0, "a row's lanes must fit the block");
    const uint32_t t = threadIdx.x;
    const uint32_t rib = t / G;
    const uint32_t lane = t % G;
    const uint32_t j = t & 15u;
    const uint32_t row0 = xcd_chunked_block(blockIdx.x, gridDim.x) * (RPS * S);
    if (om.valid != nullptr) {
        rows = valid_rows(rows, om);
        if (row0 >= rows) return;  // every row of the block is padding
    }
    const char* base = reinterpret_cast<const char*>(src);

    uint32_t row[S], off[S];
    float lw[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        row[s] = row0 + s * RPS + rib;
        const uint32_t rc = row[s] < rows ? row[s] : rows - 1;
        off[s] = (rc * stride + lane * (SPLIT ? E / 2 : E)) * ES;
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const uint32_t rc = row[s] < rows ? row[s] : rows - 1;
        float l = -__builtin_inff();
        if (int(j) < N) {
            if (PACKED)
                l = ld_tail(base + j * plane_bytes + (rc * stride + D) * ES);
            else
                l = lse[j * lse_plane + rc];
        }
        lw[s] = l;
    }
    // The first plane group's loads go out right behind the LSE loads, so the
    // LSE round trip overlaps the data instead of preceding it (small,
    // latency-bound calls pay for exactly that) and the reductions below run
    // while the data is in flight.
    u32x4 v[PG][S];
    auto load_group = [&](int n0) {
#pragma unroll
        for (int p = 0; p < PG; ++p) {
            if (!has(n0 + p)) break;
            const char* pb = base + uint64_t(n0 + p) * plane_bytes;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                if constexpr (SPLIT) {
                    const u32x2_a4 lo = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x2_a4*>(pb + off[s]));
                    const u32x2_a4 hi = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x2_a4*>(pb + off[s] + D * ES / 2));
                    v[p][s] = u32x4{lo.x, lo.y, hi.x, hi.y};
                } else {
                    v[p][s] = PACKED ? ld16_a4_at(pb + off[s]) : ld16_nt_at(pb + off[s]);
                }
            }
        }
    };
    load_group(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float l = int(j) < N ? sanitize(lw[s]) : -__builtin_inff();
        float m = row16_max(l);
        if (m == -__builtin_inff()) m = 0.0f;
        const float w = int(j) < N ? weight(l - m, scale) : 0.0f;
        const float sum = row16_sum(w);
        lw[s] = w * (1.0f / fmaxf(sum, 1e-10f));
        if (out_lse != nullptr && lane == 0 && row[s] < rows)
            out_lse[out_row(row[s], om)] = global_lse(sum, m, inv_scale);
    }

    float acc[S][E];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int k = 0; k < E; ++k) acc[s][k] = kAccInit;
#pragma unroll 1
    for (int n0 = 0; n0 < N; n0 += PG) {
        if (n0 > 0) load_group(n0);
        __builtin_amdgcn_sched_barrier(0);  // all PG*S loads issued before the first is used
#pragma unroll
        for (int p = 0; p < PG; ++p) {
            if (!has(n0 + p)) break;
#pragma unroll
            for (int s = 0; s < S; ++s) fma_chunk<DT>(v[p][s], lane_value<G>(lw[s], n0 + p), acc[s]);
        }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        if (row[s] >= rows) continue;
        if constexpr (SPLIT) {
            float* p = static_cast<float*>(out) + uint64_t(out_row(row[s], om)) * D + lane * 4;
            st16(p, f32_chunk(acc[s][0], acc[s][1], acc[s][2], acc[s][3]));
            st16(p + D / 2, f32_chunk(acc[s][4], acc[s][5], acc[s][6], acc[s][7]));
        } else {
            store_chunk<DT>(out, uint64_t(out_row(row[s], om)) * D + lane * E, acc[s]);
        }
    }
}


// ---------------------------------------------------------------- combine (packed spans)
//
// Packed rows of 128 16-bit values (260 bytes with the fp32 LSE tail) when the
// rows are a multiple of 4 and the planes 16-byte aligned, N = 2, 4, 8 or 16.
// A wave owns four consecutive rows of every plane: a 1040-byte span, 65
// aligned 16-byte chunks. Lane i loads chunk i of each plane and every lane
// chunk 64 (one address per wave), so all loads are aligned and no separate
// LSE loads go out: the tails of rows 0, 1, 2 are dword k of the chunks of
// lanes 16, 32, 48, row 3's the last dword of chunk 64. Lane 16 k + j takes
// shard j's LSE of row k by a lane shuffle; the weights then follow the
// slotted kernel exactly (16-lane DPP max and sum, the same normalisation),
// and every element is accumulated in plane order, so the results are those
// of the slotted kernel bit for bit. Each dword of a chunk belongs to one row
// (rows start on dwords) and is weighted by that row's weight. Result chunk q
// of row k is span dwords 4 (16 k + q) + k .. + 3: this lane's accumulators
// from dword k on, then the next lane's first k dwords (lane 63: chunk 64's),
// fetched by one shuffle, so every store is a whole aligned 16-byte chunk.
// Measured on MI355X (N = 8, 16384 packed rows of 128 bf16): 1.5 % faster cold
// and 4 % faster warm than the slotted kernel with S = 1.
template <int DT, int NT>
__global__ __launch_bounds__(kBlock) void combine_span_kernel(
    const void* src, uint32_t spans, uint64_t plane_bytes, float scale, float inv_scale,
    void* __restrict__ out, float* __restrict__ out_lse) {
    static_assert(DT != LSEC_FP32 && NT >= 2 && NT <= 16, "16-bit rows, N compiled in");
    constexpr uint32_t kSpanIn = 1040, kSpanOut = 1024;  // 4 rows, with and without tails
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t k = lane >> 4;  // the row of most of this lane's chunk
    const uint32_t j = lane & 15u;
    const uint32_t span = xcd_chunked_block(blockIdx.x, gridDim.x) * (kBlock / 64) + threadIdx.x / 64;
    if (span >= spans) return;  // uniform per wave; no block-wide synchronisation follows
    const char* base = reinterpret_cast<const char*>(src) + uint64_t(span) * kSpanIn;
    u32x4 c[NT], e[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const char* pb = base + uint64_t(n) * plane_bytes;
        c[n] = ld16(pb + 16u * lane);
        e[n] = ld16(pb + 1024u);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Lanes 16, 32, 48 offer dword k - 1 of their chunks (the tails of rows
    // 0, 1, 2); lane 16 k + j keeps plane j's offer of row k's source lane.
    float l = -__builtin_inff();
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const uint32_t offer = lane == 16u ? c[n].x : (lane == 32u ? c[n].y : c[n].z);
        const uint32_t got = uint32_t(__shfl(int(offer), int((k + 1u) * 16u) & 63));
        const uint32_t mine = k == 3u ? e[n].w : got;
        if (j == uint32_t(n)) l = __uint_as_float(mine);
    }
    l = j < uint32_t(NT) ? sanitize(l) : -__builtin_inff();
    float m = row16_max(l);
    if (m == -__builtin_inff()) m = 0.0f;
    const float w = j < uint32_t(NT) ? weight(l - m, scale) : 0.0f;
    const float sum = row16_sum(w);
    const float wn = w * (1.0f / fmaxf(sum, 1e-10f));
    if (out_lse != nullptr && j == 0u) out_lse[uint64_t(span) * 4u + k] = global_lse(sum, m, inv_scale);
    // Dword 0 of lanes 32 and 48 and dword 1 of lane 48 belong to the row
    // before the lane's own; dword k - 1 of lanes 16, 32, 48 is a tail, whose
    // accumulator is never stored. Chunk 64's first three dwords are row 3's.
    const bool prev0 = lane == 32u || lane == 48u;
    const bool prev1 = lane == 48u;
    float acc[8], acce[6];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = kAccInit;
#pragma unroll
    for (int q = 0; q < 6; ++q) acce[q] = kAccInit;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const float w_own = __shfl(wn, n, 16);
        const float w_prev = __shfl(wn, int((lane & ~15u) - 16u + uint32_t(n)) & 63);
        const float w3 = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wn), 48 + n));
        const float w0 = prev0 ? w_prev : w_own;
        const float w1 = prev1 ? w_prev : w_own;
        float a, b;
        Elem<DT>::dec2(c[n].x, a, b);
        acc[0] = fmaf(a, w0, acc[0]);
        acc[1] = fmaf(b, w0, acc[1]);
        Elem<DT>::dec2(c[n].y, a, b);
        acc[2] = fmaf(a, w1, acc[2]);
        acc[3] = fmaf(b, w1, acc[3]);
        Elem<DT>::dec2(c[n].z, a, b);
        acc[4] = fmaf(a, w_own, acc[4]);
        acc[5] = fmaf(b, w_own, acc[5]);
        Elem<DT>::dec2(c[n].w, a, b);
        acc[6] = fmaf(a, w_own, acc[6]);
        acc[7] = fmaf(b, w_own, acc[7]);
        Elem<DT>::dec2(e[n].x, a, b);
        acce[0] = fmaf(a, w3, acce[0]);
        acce[1] = fmaf(b, w3, acce[1]);
        Elem<DT>::dec2(e[n].y, a, b);
        acce[2] = fmaf(a, w3, acce[2]);
        acce[3] = fmaf(b, w3, acce[3]);
        Elem<DT>::dec2(e[n].z, a, b);
        acce[4] = fmaf(a, w3, acce[4]);
        acce[5] = fmaf(b, w3, acce[5]);
    }
    // The next lane's first three dwords (six values), or chunk 64's for lane 63.
    float nx[6];
#pragma unroll
    for (int q = 0; q < 6; ++q) {
        const float down = __shfl_down(acc[q], 1);
        nx[q] = lane == 63u ? acce[q] : down;
    }
    // Element q of the result chunk is value q + 2 k of (acc, nx).
    float r[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float r1 = q + 2 < 8 ? acc[(q + 2) & 7] : nx[(q + 2 - 8) & 7];
        const float r2 = q + 4 < 8 ? acc[(q + 4) & 7] : nx[(q + 4 - 8) & 7];
        const float r3 = q + 6 < 8 ? acc[(q + 6) & 7] : nx[(q + 6 - 8) & 7];
        r[q] = k == 0u ? acc[q] : (k == 1u ? r1 : (k == 2u ? r2 : r3));
    }
    const u32x4 res = {Elem<DT>::enc2(r[0], r[1]), Elem<DT>::enc2(r[2], r[3]),
                       Elem<DT>::enc2(r[4], r[5]), Elem<DT>::enc2(r[6], r[7])};
    st16(static_cast<char*>(out) + uint64_t(span) * kSpanOut + 16u * lane, res);
}


// ---------------------------------------------------------------- combine (packed fp32 spans)
//
// Packed rows of 128 fp32 values (516 bytes with the LSE in element 128) in
// whole spans of four rows, N = 2, 4, 8 or 16, 16-byte aligned planes: a
// 2064-byte span, 129 aligned 16-byte chunks. Lane i loads chunks i and
// 64 + i of each plane and every lane chunk 128 (one address per wave).
// Dword d of a span is element d - 129 r of row r = d / 129; the four LSEs
// are dwords 128 (chunk 32, dword 0), 257 (chunk 64, dword 1), 386 (chunk 96,
// dword 2) and 515 (chunk 128, dword 3), read by readlane, and lane 16 r + j
// keeps shard j's of row r. The weights then follow the slotted kernel exactly
// (16-lane DPP max and sum, the same normalisation); the weight of row r for
// plane n is read back from lane 16 r + n, and every element is accumulated
// in plane order, so the results are those of the slotted kernel bit for
// bit. Result chunk o of row k = o / 32 is span dwords 4 o + k .. + 3: the
// lane's own accumulators of chunk o from dword k on, then the first k dwords
// of chunk o + 1 (the next lane's; for lane 63 chunk 64's, held by lane 0,
// or chunk 128's), so every store is a whole aligned 16-byte chunk.
template <int NT>
__global__ __launch_bounds__(kBlock) void combine_span32_kernel(
    const void* src, uint32_t spans, uint64_t plane_bytes, float scale, float inv_scale,
    float* __restrict__ out, float* __restrict__ out_lse) {
    static_assert(NT >= 2 && NT <= 16, "N compiled in");
    constexpr uint32_t kSpanIn = 2064, kSpanOut = 512;  // bytes in, fp32 values out
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t k = lane >> 4;  // the row this lane's shard weight belongs to
    const uint32_t j = lane & 15u;
    const uint32_t span = xcd_chunked_block(blockIdx.x, gridDim.x) * (kBlock / 64) + threadIdx.x / 64;
    if (span >= spans) return;  // uniform per wave; no block-wide synchronisation follows
    const char* base = reinterpret_cast<const char*>(src) + uint64_t(span) * kSpanIn;
    u32x4 ca[NT], cb[NT], e[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const char* pb = base + uint64_t(n) * plane_bytes;
        ca[n] = ld16(pb + 16u * lane);
        cb[n] = ld16(pb + 1024u + 16u * lane);
        e[n] = ld16(pb + 2048u);
    }
    __builtin_amdgcn_sched_barrier(0);
    auto rl = [](uint32_t v, int src_lane) {
        return uint32_t(__builtin_amdgcn_readlane(int(v), src_lane));
    };
    float l = -__builtin_inff();
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const uint32_t t0 = rl(ca[n].x, 32), t1 = rl(cb[n].y, 0), t2 = rl(cb[n].z, 32);
        const uint32_t mine = k == 0u ? t0 : (k == 1u ? t1 : (k == 2u ? t2 : e[n].w));
        if (j == uint32_t(n)) l = __uint_as_float(mine);
    }
    l = j < uint32_t(NT) ? sanitize(l) : -__builtin_inff();
    float m = row16_max(l);
    if (m == -__builtin_inff()) m = 0.0f;
    const float w = j < uint32_t(NT) ? weight(l - m, scale) : 0.0f;
    const float sum = row16_sum(w);
    const float wn = w * (1.0f / fmaxf(sum, 1e-10f));
    if (out_lse != nullptr && j == 0u) out_lse[uint64_t(span) * 4u + k] = global_lse(sum, m, inv_scale);
    // Rows of this lane's dwords. Chunk `lane` (dwords 4 lane .. + 3): row 0
    // below lane 32, row 1 above; lane 32's dword 0 is row 0's LSE, its other
    // dwords row 1's. Chunk 64 + lane: lane 0's dwords 0 and 1 are row 1's
    // (element 127 and the LSE), 2 and 3 row 2's; row 2 up to lane 31; lane
    // 32's dwords 0 to 2 are row 2's (the LSE last), dword 3 row 3's; row 3
    // above. Chunk 128: row 3 (elements 125-127, then the LSE). LSE dwords are
    // accumulated like the others and never stored.
    const bool lo = lane < 32u;
    float acca[4], accb[4], acce[3];
#pragma unroll
    for (int q = 0; q < 4; ++q) acca[q] = accb[q] = kAccInit;
#pragma unroll
    for (int q = 0; q < 3; ++q) acce[q] = kAccInit;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const float w0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wn), n));
        const float w1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wn), 16 + n));
        const float w2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wn), 32 + n));
        const float w3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wn), 48 + n));
        const float wa0 = lane <= 32u ? w0 : w1;
        const float wa = lo ? w0 : w1;
        const float wb01 = lane == 0u ? w1 : (lane <= 32u ? w2 : w3);
        const float wb2 = lane <= 32u ? w2 : w3;
        const float wb3 = lo ? w2 : w3;
        acca[0] = fmaf(__uint_as_float(ca[n].x), wa0, acca[0]);
        acca[1] = fmaf(__uint_as_float(ca[n].y), wa, acca[1]);
        acca[2] = fmaf(__uint_as_float(ca[n].z), wa, acca[2]);
        acca[3] = fmaf(__uint_as_float(ca[n].w), wa, acca[3]);
        accb[0] = fmaf(__uint_as_float(cb[n].x), wb01, accb[0]);
        accb[1] = fmaf(__uint_as_float(cb[n].y), wb01, accb[1]);
        accb[2] = fmaf(__uint_as_float(cb[n].z), wb2, accb[2]);
        accb[3] = fmaf(__uint_as_float(cb[n].w), wb3, accb[3]);
        acce[0] = fmaf(__uint_as_float(e[n].x), w3, acce[0]);
        acce[1] = fmaf(__uint_as_float(e[n].y), w3, acce[1]);
        acce[2] = fmaf(__uint_as_float(e[n].z), w3, acce[2]);
    }
    // The first dwords of the next chunk: the next lane's, or for lane 63
    // chunk 64 (lane 0's second chunk) and chunk 128. Every shuffle runs on all
    // lanes before the selection: a lane shuffle reads 0 from a lane that is
    // switched off, so it must not sit in a branch that leaves lane 63 out.
    const bool last = lane == 63u;
    const float down0 = __shfl_down(acca[0], 1);
    const float first_b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, accb[0]), 0));
    const float na0 = last ? first_b : down0;
    float nb[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const float down = __shfl_down(accb[q], 1);
        nb[q] = last ? acce[q] : down;
    }
    // Chunk `lane` of the result: row 0 below lane 32 (dwords 0-3), row 1 above
    // (dwords 1-3 and the next chunk's 0). Chunk 64 + lane: row 2 below lane
    // 32 (dwords 2, 3 and the next chunk's 0, 1), row 3 above (dword 3 and the
    // next chunk's 0-2).
    const u32x4 r0 = lo ? f32_chunk(acca[0], acca[1], acca[2], acca[3])
                        : f32_chunk(acca[1], acca[2], acca[3], na0);
    const u32x4 r1 = lo ? f32_chunk(accb[2], accb[3], nb[0], nb[1])
                        : f32_chunk(accb[3], nb[0], nb[1], nb[2]);
    float* po = out + uint64_t(span) * kSpanOut;
    st16(po + 4u * lane, r0);
    st16(po + 256u + 4u * lane, r1);
}

}  // namespace

// Occupancy cap for the tiled combine, as dynamic LDS that the kernel never
// touches (a CU has 160 KB): S = 16 launches run at most 1 block per CU
// (90 KB), S = 8 at most 2 (56 KB each), S = 4 at most 4 (36 KB each). HBM
// streams better from fewer, deeper waves; measured on MI355X against the
// occupancy the registers allow: fp32 N=8 D=512 2^16 rows (S = 16, 2 blocks)
// 5.7 % faster, bf16 N=8 D=512 2^16 rows (S = 8, 3 blocks) 2.8 %, bf16 N=8
// D=128 2^17 rows (S = 4, 7 blocks) 7.0 %. The 16-bit S = 16 kernels hold
// one block per CU by their registers anyway. S <= 2 serves inputs too small
// to fill the chip, and capping it (or the pack, or the corrected partial)
// measured slower.
constexpr size_t tiled_lds_cap(int S) {
    return S == 16 ? 90000 : (S == 8 ? 56000 : (S == 4 ? 36000 : 0));
}

template <int DT, int NT, int G, bool PACKED, bool SPLIT>
void launch_tiled_s(int S, const TiledArgs& a) {
    constexpr uint32_t RPS = kBlock / G;
    const unsigned blocks = (a.rows + RPS * S - 1) / (RPS * S);
#define LSEC_TILED(SV)                                                                         \
    launch(combine_tiled_kernel<DT, NT, G, SV, PACKED, SPLIT>, dim3(blocks), dim3(kBlock),      \
           tiled_lds_cap(SV), a.st, a.src, a.lse, a.n, a.rows, a.stride, a.plane_bytes,          \
           a.lse_plane, a.scale, a.inv_scale, a.out, a.out_lse, a.om)
    switch (S) {
        case 16: LSEC_TILED(16); break;
        case 8: LSEC_TILED(8); break;
        case 4: LSEC_TILED(4); break;
        case 2: LSEC_TILED(2); break;
        default: LSEC_TILED(1); break;
    }
#undef LSEC_TILED
}

template <int DT, int G, bool PACKED, bool SPLIT>
void launch_tiled_n(int N, int S, const TiledArgs& a) {
    switch (N) {
        case 2: launch_tiled_s<DT, 2, G, PACKED, SPLIT>(S, a); break;
        case 4: launch_tiled_s<DT, 4, G, PACKED, SPLIT>(S, a); break;
        case 8: launch_tiled_s<DT, 8, G, PACKED, SPLIT>(S, a); break;
        case 16: launch_tiled_s<DT, 16, G, PACKED, SPLIT>(S, a); break;
        default: launch_tiled_s<DT, 0, G, PACKED, SPLIT>(S, a); break;  // 2 < N < 16, at run time
    }
}

template <int DT, bool PACKED, bool SPLIT>
void launch_tiled_d(int N, int S, int D, const TiledArgs& a) {
    constexpr int E = Elem<DT>::kEpc;
    switch (D) {
        case 128: launch_tiled_n<DT, 128 / E, PACKED, SPLIT>(N, S, a); break;
        case 256: launch_tiled_n<DT, 256 / E, PACKED, SPLIT>(N, S, a); break;
        default: launch_tiled_n<DT, 512 / E, PACKED, SPLIT>(N, S, a); break;
    }
}

// 16-bit partials with an fp32 result take the split-load variant.
template <int DT, bool PACKED>
void launch_tiled(int N, int S, int D, const TiledArgs& a) {
    if constexpr (DT != LSEC_FP32) {
        if (a.out_f32) {
            launch_tiled_d<DT, PACKED, true>(N, S, D, a);
            return;
        }
    }
    launch_tiled_d<DT, PACKED, false>(N, S, D, a);
}

template void launch_tiled<LSEC_TILED_DT, false>(int, int, int, const TiledArgs&);
template void launch_tiled<LSEC_TILED_DT, true>(int, int, int, const TiledArgs&);

// Packed rows of 128 values in whole spans of four: combine_span_kernel for
// 16-bit elements, combine_span32_kernel for fp32.
template <int DT>
void launch_span(int N, const TiledArgs& a) {
    const uint32_t spans = a.rows / 4;
    const unsigned blocks = (spans + kBlock / 64 - 1) / (kBlock / 64);
    if constexpr (DT != LSEC_FP32) {
#define LSEC_SPAN(NV)                                                                        \
    launch(combine_span_kernel<DT, NV>, dim3(blocks), dim3(kBlock), 0, a.st, a.src, spans,     \
           a.plane_bytes, a.scale, a.inv_scale, a.out, a.out_lse)
        switch (N) {
            case 2: LSEC_SPAN(2); break;
            case 4: LSEC_SPAN(4); break;
            case 8: LSEC_SPAN(8); break;
            default: LSEC_SPAN(16); break;
        }
#undef LSEC_SPAN
    } else {
        float* out = static_cast<float*>(a.out);
#define LSEC_SPAN32(NV)                                                                      \
    launch(combine_span32_kernel<NV>, dim3(blocks), dim3(kBlock), 0, a.st, a.src, spans,       \
           a.plane_bytes, a.scale, a.inv_scale, out, a.out_lse)
        switch (N) {
            case 2: LSEC_SPAN32(2); break;
            case 4: LSEC_SPAN32(4); break;
            case 8: LSEC_SPAN32(8); break;
            default: LSEC_SPAN32(16); break;
        }
#undef LSEC_SPAN32
    }
}

template void launch_span<LSEC_TILED_DT>(int, const TiledArgs&);

}  // namespace lsec_detail
