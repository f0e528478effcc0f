// hbm_copy.hip -- a plain streaming copy, the measuring stick for the decode.
//
// The decode is bound by HBM traffic; its roofline fraction is quoted against
// the published 8 TB/s of MI355X and against what a plain copy of known size
// reaches on the same device.  This kernel is that copy: every lane moves
// 16-byte units with dwordx4 buffer loads and stores, four units in flight
// per lane per step (lane-contiguous within a step, so a wave reads and writes
// 1 KiB contiguous runs), in a persistent grid that strides over the buffer.
// The loads and stores carry the same non-temporal hint as the decode's
// streaming planes.  Its FETCH_SIZE / WRITE_SIZE counters, read for a copy of
// known size, also calibrate the decode's traffic counters.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ecf8.h"

namespace {

constexpr int kCopyLanes = 256;
constexpr int kCopyUnroll = 4;                       // 16-byte units in flight per lane
constexpr int kCopyWgPerCu = 8;
constexpr int kNonTemporal = 2;

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint64_t bytes)
{
    const uint32_t nr = bytes < 0xFFFFFFFFull ? (uint32_t)bytes : 0xFFFFFFFFu;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nr, kRsrcWord3);
}

// Copies units [0, units) of 16 bytes.  A step of one workgroup covers
// kCopyLanes * kCopyUnroll consecutive units; steps are taken gridDim.x apart.
// Offsets are 32-bit inside a window of at most 2 GiB rebased per step, so
// any buffer size works.
__global__ __launch_bounds__(kCopyLanes) void hbm_copy_kernel(const uint8_t* __restrict__ src,
                                                              uint8_t* __restrict__ dst, uint64_t units)
{
    constexpr uint64_t kStep = (uint64_t)kCopyLanes * kCopyUnroll;
    const uint64_t steps = (units + kStep - 1) / kStep;
    for (uint64_t s = blockIdx.x; s < steps; s += gridDim.x) {
        const uint64_t u0 = s * kStep;
        const uint64_t left = units - u0 < kStep ? units - u0 : kStep;
        const Rsrc rs = make_rsrc(src + 16 * u0, 16 * left);
        const Rsrc rd = make_rsrc(dst + 16 * u0, 16 * left);
        u32x4 v[kCopyUnroll];
#pragma unroll
        for (int k = 0; k < kCopyUnroll; ++k)
            v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16u * (threadIdx.x + k * kCopyLanes), 0, kNonTemporal);
#pragma unroll
        for (int k = 0; k < kCopyUnroll; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(v[k], rd, 16u * (threadIdx.x + k * kCopyLanes), 0, kNonTemporal);
    }
}

// Copies the last bytes % 16 bytes, one lane per byte.
__global__ void hbm_copy_tail_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, uint32_t count)
{
    if (threadIdx.x < count) dst[threadIdx.x] = src[threadIdx.x];
}

}  // namespace

extern "C" int ecf8_hbm_copy(const void* src, void* dst, uint64_t bytes, void* hip_stream)
{
    if (bytes == 0) return ECF8_OK;
    if (!src || !dst) return ECF8_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) return ECF8_ERR_ARG;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return ECF8_ERR_HIP;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    const uint64_t units = bytes / 16;
    const uint8_t* s8 = static_cast<const uint8_t*>(src);
    uint8_t* d8 = static_cast<uint8_t*>(dst);
    if (units) {
        const uint64_t step = (uint64_t)kCopyLanes * kCopyUnroll;
        uint64_t grid = (uint64_t)(cus > 0 ? cus : 1) * kCopyWgPerCu;
        const uint64_t steps = (units + step - 1) / step;
        if (grid > steps) grid = steps;
        hipLaunchKernelGGL(hbm_copy_kernel, dim3((uint32_t)grid), dim3(kCopyLanes), 0, st, s8, d8, units);
    }
    const uint32_t tail = (uint32_t)(bytes & 15);
    if (tail)
        hipLaunchKernelGGL(hbm_copy_tail_kernel, dim3(1), dim3(64), 0, st, s8 + 16 * units, d8 + 16 * units, tail);
    return hipGetLastError() == hipSuccess ? ECF8_OK : ECF8_ERR_HIP;
}
