// ecf8_encode.hip -- GPU histogram and encode of FP8 E4M3 tensors (gfx950).
//
// Method (ECF8 technical blog, codearts.csdn.net): §3.1.1 (histogram of the
// exponent field, per-tensor Huffman code, exponent replaced by its codeword,
// sign and mantissa kept raw); §3.2.1 (the stream is cut into per-lane chunks
// that each carry the offset of their first codeword start, the gap, and
// blocks of lanes that carry their first output position).  The device encode
// writes exactly the bytes of the host encoder (include/ecf8.h): canonical
// codes MSB-first, nibble plane (s << 3) | m with the even element low, 4-bit
// gaps with T counted as a codeword start, uint64 block offsets.
//
// Structure (n elements, tiles of 4096 = 256 lanes x 16 elements):
//   1. tile sums of code lengths;
//   2. three small launches scan the tile sums into 64-bit tile bit offsets
//      (group totals over 4096 tiles, one workgroup scanning the group totals,
//      each group rescanning its tiles);
//   3. per tile: lane and workgroup scans give each element's bit position
//      p; codewords are OR-ed into an LDS image of the tile's bit range and
//      written out as 32-bit words (the first and last word of a tile, which
//      neighbouring tiles share, with global atomic ORs on the zeroed
//      stream); each element whose bit interval (p, p + len] holds a chunk
//      start sets that chunk's gap (p + len - start), and likewise a block
//      start sets the block offset; the nibble plane is written per lane.
//      Chunks are at least 32 bits and codewords at most 16, so an interval
//      holds at most one chunk start; a lane finds them by carrying its
//      offset inside the current chunk.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "ecf8.h"

namespace {

constexpr int kEncLanes = 256;
constexpr int kEncPerLane = 16;
constexpr uint64_t kTile = (uint64_t)kEncLanes * kEncPerLane;   // 4096 elements
constexpr int kTileWords = (int)(kTile * ECF8_MAX_CODE_LEN / 32) + 2;   // LDS bit image
constexpr int kScanLanes = 1024;
constexpr uint64_t kGroupTiles = 4ull * kScanLanes;                  // tiles per scan group

// Code table for the kernels: length and MSB-first code per symbol.
struct EncTable {
    uint32_t code[ECF8_NSYM];
    uint32_t len[ECF8_NSYM];
};

struct EncArgs {
    const uint8_t* fp8;
    uint64_t n;
    uint64_t n_blocks;
    uint32_t chunk_bits;       // 8 * C
    uint32_t tb;               // chunks per block
    uint64_t gap_count;        // chunks with a gap entry (n_blocks * TB)
    uint64_t stream_words;     // stream_bytes / 4
    uint8_t* stream;
    uint8_t* nibbles;
    uint32_t* gaps;            // 4-byte words of the gap array
    uint64_t* blk_off;
    const uint32_t* tile_sum;
    const uint64_t* tile_off;
};

__device__ __forceinline__ uint32_t load_byte(const uint8_t* p, uint64_t i, uint64_t n)
{
    return i < n ? (uint32_t)p[i] : 0u;
}

// Load the lane's 16 bytes (elements e0 .. e0 + 15), zero past n.
__device__ __forceinline__ void load16(const uint8_t* p, uint64_t e0, uint64_t n, uint32_t (&b)[kEncPerLane])
{
    if (e0 + kEncPerLane <= n && ((uintptr_t)(p + e0) & 15) == 0) {
        const uint4 v = *reinterpret_cast<const uint4*>(p + e0);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < kEncPerLane; ++i) b[i] = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
    } else {
#pragma unroll
        for (int i = 0; i < kEncPerLane; ++i) b[i] = load_byte(p, e0 + i, n);
    }
}

__global__ __launch_bounds__(256) void ecf8_zero_kernel(uint32_t* p, uint64_t words)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// Exponent histogram.  Every lane counts into its own 16 LDS bins (bin s of
// lane j at s * 256 + j: the lanes of a wave hit 64 distinct banks), then
// each bin is summed over the 256 lanes and added once to the global count.
__global__ __launch_bounds__(256) void ecf8_hist_kernel(const uint8_t* __restrict__ fp8, uint64_t n,
                                                        unsigned long long* __restrict__ freq)
{
    __shared__ uint32_t bins[ECF8_NSYM * kEncLanes];
    const int tid = threadIdx.x;
#pragma unroll
    for (int s = 0; s < ECF8_NSYM; ++s) bins[s * kEncLanes + tid] = 0u;
    const uint64_t stride = (uint64_t)gridDim.x * kTile;
    for (uint64_t e0 = (uint64_t)blockIdx.x * kTile + (uint64_t)tid * kEncPerLane; e0 < n; e0 += stride) {
        uint32_t b[kEncPerLane];
        load16(fp8, e0, n, b);
#pragma unroll
        for (int i = 0; i < kEncPerLane; ++i)
            if (e0 + i < n) bins[((b[i] >> 3) & 15u) * kEncLanes + tid] += 1u;
    }
    __syncthreads();
    // 16 lanes per bin, each summing 16 entries, then a 16-lane reduction
    const int bin = tid >> 4, part = tid & 15;
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += bins[bin * kEncLanes + part * 16 + k];
    for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off, 16);
    if (part == 0 && s) atomicAdd(&freq[bin], (unsigned long long)s);
}

// Step 1: code-length sum of each tile.
__global__ __launch_bounds__(256) void ecf8_tile_sum_kernel(EncArgs a, EncTable tab, uint32_t* __restrict__ tile_sum)
{
    __shared__ uint32_t part[4];
    __shared__ uint32_t s_len[ECF8_NSYM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < ECF8_NSYM) s_len[tid] = tab.len[tid];
    __syncthreads();
    const uint64_t tile = blockIdx.x;
    const uint64_t e0 = tile * kTile + (uint64_t)tid * kEncPerLane;
    uint32_t b[kEncPerLane];
    load16(a.fp8, e0, a.n, b);
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < kEncPerLane; ++i)
        if (e0 + i < a.n) s += s_len[(b[i] >> 3) & 15u];
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) part[wave] = s;
    __syncthreads();
    if (tid == 0) tile_sum[tile] = part[0] + part[1] + part[2] + part[3];
}

// Sum of the four tile sums a scan lane owns (zero past the last tile).
__device__ __forceinline__ uint32_t lane_tiles(const uint32_t* __restrict__ tile_sum, uint64_t tiles, uint64_t t0,
                                               uint32_t (&v)[4])
{
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[k] = t0 + k < tiles ? tile_sum[t0 + k] : 0u;
        s += v[k];
    }
    return s;
}

// Inclusive scan over a 1024-lane workgroup (64-bit), `wsum` 16 entries of LDS.
__device__ __forceinline__ uint64_t block_incl_scan(uint64_t v, uint64_t* wsum)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int off = 1; off < 64; off <<= 1) {
        const uint64_t t = __shfl_up(v, off);
        if (lane >= off) v += t;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    uint64_t before = 0;
    for (int w = 0; w < kScanLanes / 64; ++w) before += w < wave ? wsum[w] : 0ull;
    return v + before;
}

// Step 2a: total of each group of 4096 tiles.
__global__ __launch_bounds__(kScanLanes) void ecf8_group_sum_kernel(const uint32_t* __restrict__ tile_sum,
                                                                    uint64_t tiles, uint64_t* __restrict__ gsum)
{
    __shared__ uint64_t wsum[kScanLanes / 64];
    uint32_t v[4];
    const uint64_t s = lane_tiles(tile_sum, tiles, blockIdx.x * kGroupTiles + 4ull * threadIdx.x, v);
    const uint64_t incl = block_incl_scan(s, wsum);
    if (threadIdx.x == kScanLanes - 1) gsum[blockIdx.x] = incl;
}

// Step 2b: exclusive scan of the group totals in place (one workgroup; each
// lane owns a contiguous run of groups).
__global__ __launch_bounds__(kScanLanes) void ecf8_group_scan_kernel(uint64_t* __restrict__ g, uint64_t groups)
{
    __shared__ uint64_t wsum[kScanLanes / 64];
    const uint64_t per = (groups + kScanLanes - 1) / kScanLanes;
    const uint64_t lo = (uint64_t)threadIdx.x * per, hi = lo + per < groups ? lo + per : groups;
    uint64_t s = 0;
    for (uint64_t i = lo; i < hi; ++i) s += g[i];
    uint64_t run = block_incl_scan(s, wsum) - s;
    for (uint64_t i = lo; i < hi; ++i) {
        const uint64_t x = g[i];
        g[i] = run;
        run += x;
    }
}

// Step 2c: tile bit offsets = group offset + exclusive scan inside the group.
__global__ __launch_bounds__(kScanLanes) void ecf8_tile_off_kernel(const uint32_t* __restrict__ tile_sum,
                                                                   uint64_t tiles, const uint64_t* __restrict__ goff,
                                                                   uint64_t* __restrict__ tile_off)
{
    __shared__ uint64_t wsum[kScanLanes / 64];
    uint32_t v[4];
    const uint64_t t0 = blockIdx.x * kGroupTiles + 4ull * threadIdx.x;
    const uint64_t s = lane_tiles(tile_sum, tiles, t0, v);
    uint64_t run = goff[blockIdx.x] + block_incl_scan(s, wsum) - s;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (t0 + k < tiles) tile_off[t0 + k] = run;
        run += v[k];
    }
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane)
{
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(v, off);
        if (lane >= off) v += t;
    }
    return v;
}

// Step 3: encode one tile.
__global__ __launch_bounds__(256) void ecf8_encode_kernel(EncArgs a, EncTable tab)
{
    __shared__ uint32_t img[kTileWords];
    __shared__ uint32_t wsum[4];
    __shared__ uint32_t s_len[ECF8_NSYM], s_code[ECF8_NSYM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < ECF8_NSYM) {
        s_len[tid] = tab.len[tid];
        s_code[tid] = tab.code[tid];
    }
    __syncthreads();
    const uint64_t tile = blockIdx.x;
    const uint64_t e0 = tile * kTile + (uint64_t)tid * kEncPerLane;
    const uint64_t P0 = a.tile_off[tile];              // first bit of the tile
    const uint32_t S = a.tile_sum[tile];               // bits of the tile
    const uint64_t W0 = P0 >> 5;                       // first stream word of the tile
    const uint32_t nwords = (uint32_t)(((P0 + S + 31) >> 5) - W0);

    for (uint32_t i = tid; i < nwords; i += kEncLanes) img[i] = 0u;

    uint32_t b[kEncPerLane];
    load16(a.fp8, e0, a.n, b);
    uint32_t len[kEncPerLane], acc = 0;
#pragma unroll
    for (int i = 0; i < kEncPerLane; ++i) {
        len[i] = e0 + i < a.n ? s_len[(b[i] >> 3) & 15u] : 0u;
        acc += len[i];
    }
    const uint32_t incl = wave_incl_scan(acc, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) before += w < wave ? wsum[w] : 0u;
    uint32_t rel = (uint32_t)(P0 & 31) + before + incl - acc;   // bit offset inside the tile image

    // nibble plane: (s << 3) | m, even element in the low nibble
    if (e0 < a.n) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            lo |= ((((b[i] >> 4) & 8u) | (b[i] & 7u)) << (4 * i));
            hi |= ((((b[8 + i] >> 4) & 8u) | (b[8 + i] & 7u)) << (4 * i));
        }
        *reinterpret_cast<uint2*>(a.nibbles + (e0 >> 1)) = make_uint2(lo, hi);
    }

    // codewords into the LDS image (big-endian bit numbering inside each
    // word); gaps and block offsets from the chunk starts in (p, p + len]
    const uint64_t p_lane = (P0 & ~31ull) + rel;       // absolute start bit of the lane's first codeword
    uint64_t t = p_lane / a.chunk_bits;                // chunk holding it
    uint32_t r = (uint32_t)(p_lane - t * a.chunk_bits);   // offset inside chunk t
    uint64_t blk = t / a.tb;                           // block of chunk t ...
    uint32_t tb = (uint32_t)(t - blk * a.tb);          // ... and its place in the block
#pragma unroll
    for (int i = 0; i < kEncPerLane; ++i) {
        const uint32_t l = len[i];
        if (l) {
            const uint32_t code = s_code[(b[i] >> 3) & 15u];
            const uint64_t v = (uint64_t)code << (64 - l - (rel & 31));
            const uint32_t wi = rel >> 5;
            atomicOr(&img[wi], (uint32_t)(v >> 32));
            if ((uint32_t)v) atomicOr(&img[wi + 1], (uint32_t)v);
            rel += l;
            r += l;
            if (r >= a.chunk_bits) {                   // chunk t + 1 starts in (p, p + l]
                r -= a.chunk_bits;                     // its gap: next codeword start - chunk start
                ++t;
                if (++tb == a.tb) {
                    tb = 0;
                    ++blk;
                    if (blk <= a.n_blocks) a.blk_off[blk] = e0 + i + 1;
                }
                if (r && t < a.gap_count) atomicOr(&a.gaps[t >> 3], r << (4 * (uint32_t)(t & 7)));
            }
        }
    }
    __syncthreads();

    // tile image -> stream (bytes MSB-first: store each big-endian word
    // byte-swapped); words past the stream (a meta that undercounts T) are
    // dropped
    uint32_t* const out = reinterpret_cast<uint32_t*>(a.stream);
    for (uint32_t i = tid; i < nwords; i += kEncLanes) {
        if (W0 + i >= a.stream_words) break;
        const uint32_t w = __builtin_bswap32(img[i]);
        if (i == 0 || i == nwords - 1) {
            if (w) atomicOr(&out[W0 + i], w);
        } else {
            out[W0 + i] = w;
        }
    }
    if (tile == 0 && tid == 0) {
        a.blk_off[0] = 0;
        a.blk_off[a.n_blocks] = a.n;
    }
}

int check(hipError_t e) { return e == hipSuccess ? ECF8_OK : ECF8_ERR_HIP; }

// Workspace: tile sums (u32) | tile offsets (u64) | group totals/offsets (u64),
// each part 256-byte aligned.
struct EncWorkspace {
    uint64_t tiles, groups, sum_off, off_off, group_off, bytes;
};

EncWorkspace enc_workspace(uint64_t n)
{
    auto round = [](uint64_t x) { return (x + 255) / 256 * 256; };
    EncWorkspace w;
    w.tiles = (n + kTile - 1) / kTile;
    w.groups = (w.tiles + kGroupTiles - 1) / kGroupTiles;
    w.sum_off = 0;
    w.off_off = round(w.tiles * 4);
    w.group_off = w.off_off + round(w.tiles * 8);
    w.bytes = w.group_off + round(w.groups * 8) + 256;
    return w;
}

}  // namespace

extern "C" int ecf8_histogram_device(const uint8_t* fp8, uint64_t n, uint64_t* freq, void* hip_stream)
{
    if ((!fp8 && n) || !freq || ((uintptr_t)freq & 7)) return ECF8_ERR_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    hipLaunchKernelGGL(ecf8_zero_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<uint32_t*>(freq),
                       (uint64_t)2 * ECF8_NSYM);
    if (n) {
        const uint64_t tiles = (n + kTile - 1) / kTile;
        const uint64_t grid = tiles < 2048 ? tiles : 2048;
        hipLaunchKernelGGL(ecf8_hist_kernel, dim3((uint32_t)grid), dim3(256), 0, st, fp8, n,
                           reinterpret_cast<unsigned long long*>(freq));
    }
    return check(hipGetLastError());
}

extern "C" uint64_t ecf8_encode_workspace_bytes(uint64_t n)
{
    return enc_workspace(n).bytes;
}

extern "C" int ecf8_encode_device(const uint8_t* fp8, const ecf8_meta* meta, uint8_t* stream, uint8_t* nibbles,
                                  uint8_t* gaps, uint64_t* blk_off, void* workspace, uint64_t workspace_bytes,
                                  void* hip_stream)
{
    if (!meta) return ECF8_ERR_ARG;
    int rc = ecf8_validate_meta(meta);
    if (rc) return rc;
    const uint64_t n = meta->n;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (!stream || !blk_off || ((uintptr_t)stream & 3) || ((uintptr_t)blk_off & 7)) return ECF8_ERR_ARG;
    if (n == 0) {      // the 16 zero bytes of stream padding and blk_off[0] = 0
        hipLaunchKernelGGL(ecf8_zero_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<uint32_t*>(stream),
                           meta->stream_bytes / 4);
        hipLaunchKernelGGL(ecf8_zero_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<uint32_t*>(blk_off),
                           (uint64_t)2);
        return check(hipGetLastError());
    }
    if (!fp8 || !nibbles || !gaps || !workspace || ((uintptr_t)nibbles & 7) || ((uintptr_t)gaps & 3))
        return ECF8_ERR_ARG;
    const EncWorkspace W = enc_workspace(n);
    if (workspace_bytes < W.bytes || ((uintptr_t)workspace & 255)) return ECF8_ERR_WORKSPACE;
    if (W.tiles > 0xFFFFFFFFull || W.groups > 0xFFFFFFFFull) return ECF8_ERR_SIZE;

    ecf8_codebook cb = meta->cb;
    uint32_t code[ECF8_NSYM];
    rc = ecf8_canonical_codes(&cb, code);
    if (rc) return rc;
    EncTable tab;
    for (int s = 0; s < ECF8_NSYM; ++s) {
        tab.code[s] = code[s];
        tab.len[s] = cb.len[s];
    }
    uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
    uint32_t* tile_sum = reinterpret_cast<uint32_t*>(ws + W.sum_off);
    uint64_t* tile_off = reinterpret_cast<uint64_t*>(ws + W.off_off);
    uint64_t* group = reinterpret_cast<uint64_t*>(ws + W.group_off);
    EncArgs a;
    a.fp8 = fp8;
    a.n = n;
    a.n_blocks = meta->n_blocks;
    a.chunk_bits = 8u * meta->chunk_bytes;
    a.tb = meta->threads_per_block;
    a.gap_count = meta->n_blocks * meta->threads_per_block;
    a.stream_words = meta->stream_bytes / 4;
    a.stream = stream;
    a.nibbles = nibbles;
    a.gaps = reinterpret_cast<uint32_t*>(gaps);
    a.blk_off = blk_off;
    a.tile_sum = tile_sum;
    a.tile_off = tile_off;

    // zero the stream (shared boundary words and padding are OR-ed) and the
    // gaps (OR-ed nibbles; zero gaps are not written).  stream_bytes and
    // gap_bytes are multiples of 4 (C and TB are multiples of 4 and 64); the
    // kernel writes the whole nibble plane itself.
    hipLaunchKernelGGL(ecf8_zero_kernel, dim3(1024), dim3(256), 0, st, reinterpret_cast<uint32_t*>(stream),
                       meta->stream_bytes / 4);
    hipLaunchKernelGGL(ecf8_zero_kernel, dim3(256), dim3(256), 0, st, reinterpret_cast<uint32_t*>(gaps),
                       meta->gap_bytes / 4);
    hipLaunchKernelGGL(ecf8_tile_sum_kernel, dim3((uint32_t)W.tiles), dim3(kEncLanes), 0, st, a, tab, tile_sum);
    hipLaunchKernelGGL(ecf8_group_sum_kernel, dim3((uint32_t)W.groups), dim3(kScanLanes), 0, st, tile_sum,
                       W.tiles, group);
    hipLaunchKernelGGL(ecf8_group_scan_kernel, dim3(1), dim3(kScanLanes), 0, st, group, W.groups);
    hipLaunchKernelGGL(ecf8_tile_off_kernel, dim3((uint32_t)W.groups), dim3(kScanLanes), 0, st, tile_sum, W.tiles,
                       group, tile_off);
    hipLaunchKernelGGL(ecf8_encode_kernel, dim3((uint32_t)W.tiles), dim3(kEncLanes), 0, st, a, tab);
    return check(hipGetLastError());
}
