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
// known size, also calibrate the decode's traffic counters.  A second kernel
// streams the decode's own mix (fewer bytes read than written, each once), the
// rate a decode of that traffic could reach with no work of its own.
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

// The stream of a decode-like byte mix: output unit i (16 bytes) = input
// unit (i * m) >> 32 with m = floor(2^32 * in_units / out_units) <= 2^32, so
// the input is swept once (neighbouring lanes share its units and cache
// lines) while the output is written once.  Same grid, steps and hints as the
// copy.
__global__ __launch_bounds__(kCopyLanes) void hbm_stream_kernel(const uint8_t* __restrict__ src,
                                                                uint8_t* __restrict__ dst, uint64_t out_units,
                                                                uint64_t m)
{
    constexpr uint64_t kStep = (uint64_t)kCopyLanes * kCopyUnroll;
    const uint64_t steps = (out_units + kStep - 1) / kStep;
    for (uint64_t s = blockIdx.x; s < steps; s += gridDim.x) {
        const uint64_t u0 = s * kStep;
        const uint64_t left = out_units - u0 < kStep ? out_units - u0 : kStep;
        const uint64_t j0 = (u0 * m) >> 32;
        const uint64_t j1 = ((u0 + left - 1) * m) >> 32;          // < in_units
        const Rsrc rs = make_rsrc(src + 16 * j0, 16 * (j1 - j0 + 1));
        const Rsrc rd = make_rsrc(dst + 16 * u0, 16 * left);
        u32x4 v[kCopyUnroll];
#pragma unroll
        for (int k = 0; k < kCopyUnroll; ++k) {
            const uint64_t i = u0 + threadIdx.x + k * kCopyLanes;
            const uint32_t j = (uint32_t)(((i * m) >> 32) - j0);   // past the output's end: past the range, reads 0
            v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16u * j, 0, kNonTemporal);
        }
#pragma unroll
        for (int k = 0; k < kCopyUnroll; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(v[k], rd, 16u * (threadIdx.x + k * kCopyLanes), 0, kNonTemporal);
    }
}

uint32_t copy_grid(uint64_t units, int cus)
{
    const uint64_t step = (uint64_t)kCopyLanes * kCopyUnroll;
    uint64_t grid = (uint64_t)(cus > 0 ? cus : 1) * kCopyWgPerCu;
    const uint64_t steps = (units + step - 1) / step;
    return (uint32_t)(grid > steps ? steps : grid);
}

}  // namespace

extern "C" int ecf8_hbm_stream(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes,
                               void* hip_stream)
{
    if (write_bytes == 0) return read_bytes == 0 ? ECF8_OK : ECF8_ERR_ARG;
    if (!src || !dst || read_bytes == 0 || read_bytes > write_bytes || ((read_bytes | write_bytes) & 15))
        return ECF8_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) return ECF8_ERR_ARG;
    if (write_bytes / 16 > 0xFFFFFFFFull) return ECF8_ERR_SIZE;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return ECF8_ERR_HIP;
    const uint64_t out_units = write_bytes / 16, in_units = read_bytes / 16;
    const uint64_t m = (uint64_t)(((unsigned __int128)in_units << 32) / out_units);   // <= 2^32
    hipLaunchKernelGGL(hbm_stream_kernel, dim3(copy_grid(out_units, cus)), dim3(kCopyLanes), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), static_cast<const uint8_t*>(src),
                       static_cast<uint8_t*>(dst), out_units, m);
    return hipGetLastError() == hipSuccess ? ECF8_OK : ECF8_ERR_HIP;
}

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
