// lsec_floor.hip -- measurement aids of liblsec.so (include/lsec_floor.h): an
// empty launch, a plain streaming read and a plain copy, the reference points
// the library's kernels are timed against, and the per-thread events that
// lsec_time_next_launch arms for the next launch. Not part of the combine.
//
// Build with -Xclang -target-feature -Xclang -packed-fp32-ops (as every unit
// of the library).

#include "lsec_device.h"
#include "lsec_floor.h"

namespace lsec_detail {
namespace {

__global__ void floor_empty_kernel() {}

constexpr int kFloorLoads = 4;                                  // 16-byte loads per lane
constexpr uint64_t kFloorChunksPerBlock = uint64_t(kBlock) * kFloorLoads;  // 16 KiB

// Block b reads chunks [b * 1024, (b + 1) * 1024) of 16 bytes (the last block
// stops at n16): lane t loads chunks b * 1024 + t + 256 k, k < 4, so each of
// its four load instructions covers 4 KiB contiguous bytes per block. The
// block's XOR of the words it read goes to sink[b].
__global__ __launch_bounds__(kBlock) void floor_read_kernel(const u32x4* __restrict__ src,
                                                            uint64_t n16,
                                                            uint32_t* __restrict__ sink) {
    __shared__ uint32_t part[kBlock / 64];
    const uint64_t base = uint64_t(blockIdx.x) * kFloorChunksPerBlock + threadIdx.x;
    u32x4 v[kFloorLoads];
#pragma unroll
    for (int k = 0; k < kFloorLoads; ++k) {
        const uint64_t i = base + uint64_t(k) * kBlock;
        v[k] = i < n16 ? ld16(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < kFloorLoads; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x ^= uint32_t(__shfl_xor(int(x), d));
    if ((threadIdx.x & 63u) == 0) part[threadIdx.x / 64] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
#pragma unroll
        for (int w = 0; w < kBlock / 64; ++w) y ^= part[w];
        sink[blockIdx.x] = y;
    }
}

// Block b copies chunks [b * 1024, (b + 1) * 1024) (the last block stops at
// n16); lane t moves chunks b * 1024 + t + 256 k, k < 4, all four loads issued
// before the first store.
__global__ __launch_bounds__(kBlock) void floor_copy_kernel(const u32x4* __restrict__ src,
                                                            u32x4* __restrict__ dst, uint64_t n16) {
    const uint64_t base = uint64_t(blockIdx.x) * kFloorChunksPerBlock + threadIdx.x;
    u32x4 v[kFloorLoads];
#pragma unroll
    for (int k = 0; k < kFloorLoads; ++k) {
        const uint64_t i = base + uint64_t(k) * kBlock;
        v[k] = i < n16 ? ld16(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kFloorLoads; ++k) {
        const uint64_t i = base + uint64_t(k) * kBlock;
        if (i < n16) st16(dst + i, v[k]);
    }
}

// Events armed by lsec_time_next_launch, per calling thread.
thread_local LaunchEvents g_armed{nullptr, nullptr};

}  // namespace

LaunchEvents take_launch_events() {
    const LaunchEvents ev = g_armed;
    g_armed = LaunchEvents{nullptr, nullptr};
    return ev;
}

}  // namespace lsec_detail

using namespace lsec_detail;

extern "C" {

int lsec_time_next_launch(void* start, void* stop) {
    if ((start == nullptr) != (stop == nullptr)) return LSEC_ERR_NULL;
    g_armed = LaunchEvents{static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)};
    return LSEC_OK;
}

int lsec_floor_empty(void* stream) {
    (void)hipGetLastError();
    launch(floor_empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? LSEC_OK : LSEC_ERR_LAUNCH;
}

int64_t lsec_floor_read_blocks(int64_t bytes) {
    if (bytes < 0 || bytes % 16 != 0) return -1;
    const uint64_t n16 = uint64_t(bytes) / 16;
    return int64_t((n16 + kFloorChunksPerBlock - 1) / kFloorChunksPerBlock);
}

int lsec_floor_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    const int64_t blocks = lsec_floor_read_blocks(bytes);
    if (blocks < 0 || blocks > int64_t(UINT32_MAX)) return LSEC_ERR_SHAPE;
    if (blocks == 0) return LSEC_OK;
    if (!src || !sink) return LSEC_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return LSEC_ERR_ALIGNMENT;
    (void)hipGetLastError();
    launch(floor_read_kernel, dim3(unsigned(blocks)), dim3(kBlock), 0,
           static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), uint64_t(bytes) / 16,
           sink);
    return hipGetLastError() == hipSuccess ? LSEC_OK : LSEC_ERR_LAUNCH;
}

int lsec_floor_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    const int64_t blocks = lsec_floor_read_blocks(bytes);
    if (blocks < 0 || blocks > int64_t(UINT32_MAX)) return LSEC_ERR_SHAPE;
    if (blocks == 0) return LSEC_OK;
    if (!src || !dst) return LSEC_ERR_NULL;
    if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) != 0)
        return LSEC_ERR_ALIGNMENT;
    (void)hipGetLastError();
    launch(floor_copy_kernel, dim3(unsigned(blocks)), dim3(kBlock), 0,
           static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
           static_cast<u32x4*>(dst), uint64_t(bytes) / 16);
    return hipGetLastError() == hipSuccess ? LSEC_OK : LSEC_ERR_LAUNCH;
}

}  // extern "C"
