// lsec_device.h -- shared by the translation units of liblsec.so: element
// types, load / store helpers, the weight arithmetic, lane reductions, the
// XCD-ordered tile walk, and the interface between the host code and the
// tiled combine (compiled in its own unit per element type so that the
// library builds in parallel). Internal: not installed, not part of the C ABI.

#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsec.h"

namespace lsec_detail {

constexpr int kBlock = 256;  // a row's lanes (D / elements per chunk) must fit one block

// ---------------------------------------------------------------- helpers

// Unsigned 32-bit division by an invariant divisor d >= 1 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// q = (umulhi(x, m) + x) >> l with l = ceil(log2 d), m = 2^32 (2^l - d) / d + 1.
struct FastDiv {
    uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{d, uint32_t(m), l};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t x, FastDiv f) {
    return uint32_t((uint64_t(__umulhi(x, f.m)) + x) >> f.l);
}

// Output row order. Identity (a == 0), or the token-major transpose of the
// Ascend SFA merge with its token in the second input dimension: input row
// r = (x, t) of an [A, C] grid (x < A, t < C) is stored at output row t * A + x.
struct OutMap {
    uint32_t a;  // A, or 0 for the identity
    FastDiv c;   // divides by C
    // When set, only the rows of the first *valid tokens (rows_per_token rows
    // each) are read and written; the count lives in device memory.
    const int32_t* valid;
    uint32_t rows_per_token;
};

// The rows a launch combines: all `rows`, or those of the first *om.valid
// tokens (clamped to [0, rows]).
__device__ __forceinline__ uint32_t valid_rows(uint32_t rows, const OutMap& om) {
    if (om.valid == nullptr) return rows;
    const int32_t t = *om.valid;
    if (t <= 0) return 0;
    const uint64_t r = uint64_t(uint32_t(t)) * om.rows_per_token;
    return r < rows ? uint32_t(r) : rows;
}

__device__ __forceinline__ uint32_t out_row(uint32_t r, OutMap om) {
    if (om.a == 0) return r;
    const uint32_t x = fdiv(r, om.c);
    return (r - x * om.c.d) * om.a + x;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The same four (two) dwords at 4-byte alignment (packed rows start every
// D + P elements, i.e. on 4-byte boundaries).
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

// Every input byte is read once and every output byte written once, so all
// streaming accesses are non-temporal (the `nt` cache policy); on MI355X plain
// loads cost 12-15 % at 2 GB per call and up to 40 % on small cold calls.
// 16-byte load / store at a 16-byte aligned address.
__device__ __forceinline__ u32x4 ld16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
// 16-byte load / store at a 4-byte aligned address (packed rows): gfx950
// serves dwordx4 at dword alignment. Packed rows are written in pieces that
// straddle cache lines, so those stores keep the default policy: L2 assembles
// whole lines before they go to HBM (non-temporal stores here measured about
// 10 % slower).
__device__ __forceinline__ u32x4 ld16_a4(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_a4*>(p));
}
__device__ __forceinline__ void st16_a4(void* p, u32x4 v) {
    *reinterpret_cast<u32x4_a4*>(p) = static_cast<u32x4_a4>(v);
}
// The fp32 LSE in the tail of a packed row (same cache lines as the row).
__device__ __forceinline__ float ld_tail(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const float*>(p));
}
__device__ __forceinline__ void st_tail(void* p, float v) { *reinterpret_cast<float*>(p) = v; }

// Element types. T is the storage word; kEpc elements make one 16-byte chunk;
// kPack elements carry one fp32 LSE in a packed row. dec / enc convert to and
// from fp32 (round to nearest even).
template <int DT>
struct Elem;

template <>
struct Elem<LSEC_BF16> {
    using T = uint16_t;
    static constexpr int kEpc = 8;
    static constexpr int kPack = 2;
    __device__ static __forceinline__ void dec2(uint32_t u, float& a, float& b) {
        a = __uint_as_float(u << 16);
        b = __uint_as_float(u & 0xffff0000u);
    }
    __device__ static __forceinline__ uint32_t enc2(float a, float b) {
        bf16x2 p = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32: round to nearest even
        return __builtin_bit_cast(uint32_t, p);
    }
    __device__ static __forceinline__ float dec1(uint16_t h) {
        return __uint_as_float(uint32_t(h) << 16);
    }
    __device__ static __forceinline__ uint16_t enc1(float a) {
        return __builtin_bit_cast(uint16_t, (__bf16)a);
    }
};

template <>
struct Elem<LSEC_FP16> {
    using T = uint16_t;
    static constexpr int kEpc = 8;
    static constexpr int kPack = 2;
    __device__ static __forceinline__ void dec2(uint32_t u, float& a, float& b) {
        f16x2 h = __builtin_bit_cast(f16x2, u);
        a = (float)h.x;
        b = (float)h.y;
    }
    __device__ static __forceinline__ uint32_t enc2(float a, float b) {
        f16x2 p = {(_Float16)a, (_Float16)b};  // v_cvt_f16_f32: round to nearest even
        return __builtin_bit_cast(uint32_t, p);
    }
    __device__ static __forceinline__ float dec1(uint16_t h) {
        return (float)__builtin_bit_cast(_Float16, h);
    }
    __device__ static __forceinline__ uint16_t enc1(float a) {
        return __builtin_bit_cast(uint16_t, (_Float16)a);
    }
};

template <>
struct Elem<LSEC_FP32> {
    using T = uint32_t;
    static constexpr int kEpc = 4;
    static constexpr int kPack = 1;
    __device__ static __forceinline__ float dec1(uint32_t u) { return __uint_as_float(u); }
    __device__ static __forceinline__ uint32_t enc1(float a) { return __float_as_uint(a); }
};

// NaN and +-inf shard LSEs count as -inf (exponent field all ones).
__device__ __forceinline__ float sanitize(float l) {
    return (__float_as_uint(l) & 0x7f800000u) == 0x7f800000u ? -__builtin_inff() : l;
}

// Weight of a shard: 2^(x * scale), x = l' - m <= 0 or -inf. scale = log2(e)
// for base-e LSEs (e^x = 2^(x log2 e)) and 1 for base 2. v_exp_f32 maps -inf
// to 0. A NaN weight (not reachable: x is never NaN) would become 0.
__device__ __forceinline__ float weight(float x, float scale) {
    float w = __builtin_amdgcn_exp2f(x * scale);
    return w != w ? 0.0f : w;
}

// Global LSE: ln S + m = log2(S) ln 2 + m (base e), or log2(S) + m (base 2).
// S = 0 (all shards non-finite) gives -inf.
__device__ __forceinline__ float global_lse(float s, float m, float inv_scale) {
    return log2f(s) * inv_scale + m;
}

// Accumulators start at -0: fma(a, w, -0) is exactly a * w for every
// product, a signed zero included (starting at +0 would turn a -0 product into
// +0), so a single shard of weight 1 comes back bit for bit, -0 included.
constexpr float kAccInit = -0.0f;

// Accumulate one 16-byte chunk (kEpc elements) scaled by w into acc.
template <int DT>
__device__ __forceinline__ void fma_chunk(u32x4 v, float w, float (&acc)[Elem<DT>::kEpc]) {
    if constexpr (DT == LSEC_FP32) {
        acc[0] = fmaf(__uint_as_float(v.x), w, acc[0]);
        acc[1] = fmaf(__uint_as_float(v.y), w, acc[1]);
        acc[2] = fmaf(__uint_as_float(v.z), w, acc[2]);
        acc[3] = fmaf(__uint_as_float(v.w), w, acc[3]);
    } else {
        float a, b;
        Elem<DT>::dec2(v.x, a, b);
        acc[0] = fmaf(a, w, acc[0]);
        acc[1] = fmaf(b, w, acc[1]);
        Elem<DT>::dec2(v.y, a, b);
        acc[2] = fmaf(a, w, acc[2]);
        acc[3] = fmaf(b, w, acc[3]);
        Elem<DT>::dec2(v.z, a, b);
        acc[4] = fmaf(a, w, acc[4]);
        acc[5] = fmaf(b, w, acc[5]);
        Elem<DT>::dec2(v.w, a, b);
        acc[6] = fmaf(a, w, acc[6]);
        acc[7] = fmaf(b, w, acc[7]);
    }
}

__device__ __forceinline__ u32x4 f32_chunk(float a, float b, float c, float d) {
    u32x4 r = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
    return r;
}

// Store a lane's kEpc results at element `idx` of `out` (16-byte aligned) in
// the input dtype (fp32 inputs: fp32). An fp32 result from 16-bit partials
// does not come through here: those kernels read split halves of the row so
// that each of a lane's two 16-byte fp32 stores belongs to an instruction
// writing one contiguous half of the row (two stores covering every other 16
// bytes of a wave's span had L2 write 17-18 % more than the result holds with
// non-temporal stores, and ran slower with the default policy).
template <int DT>
__device__ __forceinline__ void store_chunk(void* out, uint64_t idx,
                                            const float (&acc)[Elem<DT>::kEpc]) {
    if constexpr (DT == LSEC_FP32) {
        st16(static_cast<float*>(out) + idx, f32_chunk(acc[0], acc[1], acc[2], acc[3]));
    } else {
        u32x4 r = {Elem<DT>::enc2(acc[0], acc[1]), Elem<DT>::enc2(acc[2], acc[3]),
                   Elem<DT>::enc2(acc[4], acc[5]), Elem<DT>::enc2(acc[6], acc[7])};
        st16(static_cast<uint16_t*>(out) + idx, r);
    }
}

// One result element (general paths).
template <int DT>
__device__ __forceinline__ void store_elem(void* out, int64_t idx, float v, int out_f32) {
    if (DT == LSEC_FP32 || out_f32)
        static_cast<float*>(out)[idx] = v;
    else
        static_cast<typename Elem<DT>::T*>(out)[idx] = Elem<DT>::enc1(v);
}

// ---------------------------------------------------------------- lane reductions (tiled kernels)

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

// Reductions over the 16 lanes of each DPP row (every lane gets the result).
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_mov<0x128>(v));  // row_ror:8
    v = fmaxf(v, dpp_mov<0x124>(v));  // row_ror:4
    v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm:[2,3,0,1]
    v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm:[1,0,3,2]
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0x128>(v);
    v += dpp_mov<0x124>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0xB1>(v);
    return v;
}

// Value held by lane n of this lane's 16-lane segment (n uniform). With
// G >= 64 every lane of a wave belongs to the same row, and each 16-lane
// segment holds the same values, so lane n of the wave is lane n of the
// segment.
template <int G>
__device__ __forceinline__ float lane_value(float v, int n) {
    if constexpr (G >= 64)
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), n));
    else
        return __shfl(v, n, 16);
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on
// XCD i mod 8). Remap so that each XCD takes chunks of kXcdChunk consecutive
// tiles: logical tile = (chunk * 8 + xcd) * kXcdChunk + index within chunk.
// The remap is a permutation of [0, nblocks): the grid's tail that does not
// fill a whole round of 8 chunks keeps the identity. Measured on MI355X: 4-8 %
// more bandwidth for the streaming combine than plain round-robin order.
constexpr uint32_t kXcdChunk = 16;

__device__ __forceinline__ uint32_t xcd_chunked_block(uint32_t bid, uint32_t nblocks) {
    const uint32_t full = nblocks / (8 * kXcdChunk) * (8 * kXcdChunk);
    if (bid >= full) return bid;
    const uint32_t xcd = bid % 8, i = bid / 8;
    return ((i / kXcdChunk) * 8 + xcd) * kXcdChunk + i % kXcdChunk;
}

// ---------------------------------------------------------------- kernel launch
//
// Every kernel of the library is launched through launch(): a plain launch on
// the caller's stream, unless the calling thread has armed a pair of events
// with the measurement aid lsec_time_next_launch (lsec_floor.h). Then this
// launch records its kernel's start and end in them (hipExtLaunchKernelGGL,
// whose timestamps come from the kernel's own dispatch, without separate
// event markers around it) and the pair is disarmed.
struct LaunchEvents {
    hipEvent_t start, stop;
};

// The armed pair of the calling thread (nulls if none); disarms it.
// Defined with the measurement aids (lsec_floor.hip).
LaunchEvents take_launch_events();

template <typename... P, typename... A>
inline void launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem, hipStream_t st,
                   A... args) {
    const LaunchEvents ev = take_launch_events();
    if (ev.start != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, uint32_t(shmem), st, ev.start, ev.stop, 0u,
                              args...);
    else
        kernel<<<grid, block, shmem, st>>>(args...);
}

// ---------------------------------------------------------------- host interface of the tiled combine

struct TiledArgs {
    const void* src;
    const float* lse;
    int n;
    uint32_t rows, stride;
    uint64_t plane_bytes;
    uint32_t lse_plane;
    float scale, inv_scale;
    void* out;
    int out_f32;
    float* out_lse;
    OutMap om;
    hipStream_t st;
};

// Launches the tiled combine (lsec_tiled.hip, one unit per element type DT):
// N in [2, 16], S in {16, 8, 4, 2, 1}, D in {128, 256, 512}; an fp32 result
// from 16-bit partials when a.out_f32.
template <int DT, bool PACKED>
void launch_tiled(int N, int S, int D, const TiledArgs& a);

// Launches the span combine of packed rows (lsec_tiled.hip): D = 128, N in
// {2, 4, 8, 16}, a.rows a multiple of 4, a.src 16-byte aligned, identity
// output order, no valid count, a result in the input dtype (16-bit or fp32).
template <int DT>
void launch_span(int N, const TiledArgs& a);

}  // namespace lsec_detail
