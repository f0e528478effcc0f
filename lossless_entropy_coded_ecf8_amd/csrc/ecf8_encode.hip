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
// Two passes over the input, in tiles of 4096 elements (256 lanes x 16):
//   1. histogram: per tile, the count of each of the 16 exponent symbols
//      (kept in the workspace as 16-bit fields) and the tensor's totals;
//   -- the host turns the totals into code lengths and sizes --
//   2. three small launches turn the per-tile counts and the code lengths
//      into 64-bit tile bit offsets (tile bits = sum of count x length;
//      group totals over 1024 tiles, one workgroup scanning the group
//      totals, each group rescanning its tiles), clear the stream words that
//      two tiles share, and write a 256-entry table of codeword pairs;
//   3. encode, one workgroup per tile: a lane looks up its 8 element pairs
//      in the pair table, lane and workgroup scans give the bit positions,
//      each pair is OR-ed into an LDS image of the tile's bit range, and the
//      image goes out as 32-bit words (the first and last word of the tile,
//      when shared with a neighbouring tile, with a global atomic OR on the
//      cleared word); each chunk start inside a lane's bit range gives that
//      chunk's gap (next codeword start - chunk start) into an LDS gap image,
//      written out as whole words, and a block start the block offset; the
//      nibble plane is written per lane.  Chunks are at least 32 bits and
//      codewords at most 16, so an element's bit interval holds at most one
//      chunk start.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "ecf8.h"

namespace {

constexpr int kEncLanes = 256;
constexpr int kEncPerLane = 16;
constexpr uint64_t kTile = (uint64_t)kEncLanes * kEncPerLane;          // 4096 elements
constexpr int kTileWords = (int)(kTile * ECF8_MAX_CODE_LEN / 32) + 2;  // LDS bit image
// LDS gap image: a tile's bits span at most kTileWords * 32 bits, so (chunks
// being >= 32 bits) at most kTileWords + 1 chunk starts, 8 gaps per word.
constexpr int kGapWords = (kTileWords + 1) / 8 + 3;
constexpr int kScanLanes = 256;                                        // lanes of the per-group scans
constexpr uint64_t kGroupTiles = 4ull * kScanLanes;                    // tiles per scan group
constexpr int kCountWords = 8;                                         // per-tile counts: 16 x 16 bits
constexpr int kHistWaves = 4;                                          // histogram: one tile per wave at a time
constexpr int kHistLoads = (int)(kTile / 64 / 16);                     // 16-byte loads per lane per tile

// Symbol counted by 16-bit field f (0 = low half) of per-tile count word d.
__host__ __device__ constexpr int count_symbol(int d, int f) { return (d >> 1) + 4 * (2 * (d & 1) + f); }

// Code table for the encode kernel: length and MSB-first code per symbol.
struct EncTable {
    uint32_t code[ECF8_NSYM];
    uint32_t len[ECF8_NSYM];
};

// Code length of the symbol of each count field: v[2d + f] for word d, half f.
struct CountLens {
    uint32_t v[2 * kCountWords];
};

struct EncArgs {
    const uint8_t* fp8;
    uint64_t n;
    uint64_t tiles;
    uint64_t n_blocks;
    uint32_t chunk_bits;       // 8 * C
    uint32_t tb;               // chunks per block
    uint64_t gap_count;        // chunks with a gap entry (n_blocks * TB)
    uint64_t gap_words;        // gap_bytes / 4
    uint64_t stream_words;     // stream_bytes / 4
    uint32_t* stream;
    uint8_t* nibbles;
    uint32_t* gaps;            // 4-byte words of the gap array
    uint64_t* blk_off;
    const uint64_t* tile_off;  // tiles + 1 entries; tile_off[tiles] = T
    const uint64_t* tile_chunk;   // per tile and for T: chunk holding bit tile_off & ~31, and its block
    const uint2* pairs;        // codeword-pair table, 256 entries
    uint32_t* side;            // per tile: its partial first and last stream words, first and last gap words
    uint64_t m_chunk;          // ceil(2^40 / chunk_bits)
    uint64_t m_tb;             // ceil(2^40 / tb)
};

// x / d for x < 2^20 and d <= 1024 through m = ceil(2^40 / d): the product's
// error is below x / 2^40 < 1 / d, so the quotient is exact.
__device__ __forceinline__ uint32_t div_small(uint32_t x, uint64_t m) { return (uint32_t)(((uint64_t)x * m) >> 40); }

// The lane's 16 bytes (elements e0 .. e0 + 15) as 4 little-endian words, zero past n.
__device__ __forceinline__ void load16(const uint8_t* p, uint64_t e0, uint64_t n, uint32_t (&w)[4])
{
    if (e0 + kEncPerLane <= n && ((uintptr_t)(p + e0) & 15) == 0) {
        const uint4 v = *reinterpret_cast<const uint4*>(p + e0);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    } else {            // ragged tail or unaligned input: byte loads at clamped addresses (n >= 1)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t x = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint64_t i = e0 + 4 * q + k;
                const uint32_t v = p[i < n ? i : n - 1];
                x |= (i < n ? v : 0u) << (8 * k);
            }
            w[q] = x;
        }
    }
}

__global__ __launch_bounds__(256) void ecf8_zero_kernel(uint32_t* p, uint64_t words)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// Sum of v over the 64 lanes of the wave (uniform): DPP row shifts leave each
// 16-lane row's total in its last lane; the four row totals are read out.
__device__ __forceinline__ uint32_t wave_total(uint32_t v)
{
    v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    return __builtin_amdgcn_readlane(v, 15) + __builtin_amdgcn_readlane(v, 31) + __builtin_amdgcn_readlane(v, 47) +
           __builtin_amdgcn_readlane(v, 63);
}

// One tile's histogram by one wave: lane `lane` holds elements
// k * 1024 + 16 lane + i (k < 4, i < 16) of the tile in w; `pad` of them are
// zero bytes past n, counted as symbol 0 and taken off.  Per lane the counts
// go to 4-bit fields (16 elements), then 8-bit fields (64 elements); the
// tile's 8 count words (16-bit fields, count_symbol order) come from one DPP
// reduction each and are wave-uniform.
__device__ __forceinline__ void tile_hist(const uint32_t (&w)[kHistLoads][4], uint32_t pad, uint32_t (&c)[kCountWords])
{
    const uint64_t m8 = 0x0F0F0F0F0F0F0F0Full, m16 = 0x00FF00FF00FF00FFull;
    uint64_t even = 0, odd = 0;                           // byte j: count of symbol 2j / 2j + 1
#pragma unroll
    for (int k = 0; k < kHistLoads; ++k) {
        uint64_t A = 0, B = 0;                            // 4-bit fields, elements 0..7 and 8..15
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t e = w[k][q] & 0x78787878u;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t sh = (e >> (8 * b + 1)) & 63u;   // 4 x symbol
                if (q < 2)
                    A += 1ull << sh;
                else
                    B += 1ull << sh;
            }
        }
        even += (A & m8) + (B & m8);
        odd += ((A >> 4) & m8) + ((B >> 4) & m8);
    }
    const uint64_t r[4] = {(even & m16) - pad, odd & m16, (even >> 8) & m16, (odd >> 8) & m16};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        c[2 * q] = wave_total((uint32_t)r[q]);
        c[2 * q + 1] = wave_total((uint32_t)(r[q] >> 32));
    }
}

// Pass 1: exponent histogram.  Each wave takes whole tiles (grid-stride), 64
// elements per lane in four coalesced 16-byte loads, the next tile's loads
// issued before the current one is counted; the tile's counts are stored (if
// tile_counts is given) and added to the wave's uniform running totals.  A
// ragged last tile, or every tile of an input that is not 16-byte aligned,
// takes a second loop with bounds-checked loads.  No barrier until the end,
// where the four waves' totals meet in LDS and go to the global counts.
__global__ __launch_bounds__(256) void ecf8_hist_kernel(const uint8_t* __restrict__ fp8, uint64_t n, uint64_t tiles,
                                                        unsigned long long* __restrict__ freq,
                                                        uint32_t* __restrict__ tile_counts)
{
    __shared__ uint64_t fold[kHistWaves][ECF8_NSYM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint64_t tot[ECF8_NSYM];                              // wave-uniform running totals, count-field order
#pragma unroll
    for (int i = 0; i < ECF8_NSYM; ++i) tot[i] = 0;
    auto account = [&](uint64_t t, const uint32_t (&c)[kCountWords]) {
        if (tile_counts && lane == 0) {
            uint4* dst = reinterpret_cast<uint4*>(tile_counts + t * kCountWords);
            dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
            dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
        }
#pragma unroll
        for (int d = 0; d < kCountWords; ++d) {
            tot[2 * d] += c[d] & 0xFFFFu;
            tot[2 * d + 1] += c[d] >> 16;
        }
    };
    const uint64_t stride = (uint64_t)gridDim.x * kHistWaves;
    const uint64_t first = (uint64_t)blockIdx.x * kHistWaves + wave;
    const uint64_t full = ((uintptr_t)fp8 & 15) == 0 ? n / kTile : 0;   // tiles read with plain vector loads
    const uint32_t lane_off = (uint32_t)lane * kEncPerLane;
    uint64_t t = first;
    uint4 nx[kHistLoads];
    auto load_full = [&](uint64_t tt) {
        const uint64_t s = tt < full ? tt : 0;            // past the last full tile: tile 0 again (discarded)
#pragma unroll
        for (int k = 0; k < kHistLoads; ++k)
            nx[k] = *reinterpret_cast<const uint4*>(fp8 + s * kTile + k * (64 * kEncPerLane) + lane_off);
    };
    if (t < full) load_full(t);
    for (; t < full; t += stride) {
        uint32_t w[kHistLoads][4];
#pragma unroll
        for (int k = 0; k < kHistLoads; ++k) {
            w[k][0] = nx[k].x;
            w[k][1] = nx[k].y;
            w[k][2] = nx[k].z;
            w[k][3] = nx[k].w;
        }
        if (t + stride < full) load_full(t + stride);
        uint32_t c[kCountWords];
        tile_hist(w, 0u, c);
        account(t, c);
    }
    // the rest (a ragged last tile; all tiles of an unaligned input)
    for (t = full + ((first + stride - full % stride) % stride); t < tiles; t += stride) {
        uint32_t w[kHistLoads][4];
        uint32_t pad = 0;
#pragma unroll
        for (int k = 0; k < kHistLoads; ++k) {
            const uint64_t e0 = t * kTile + (uint64_t)k * (64 * kEncPerLane) + lane_off;
            load16(fp8, e0, n, w[k]);
            pad += e0 >= n ? kEncPerLane : (e0 + kEncPerLane > n ? (uint32_t)(e0 + kEncPerLane - n) : 0u);
        }
        uint32_t c[kCountWords];
        tile_hist(w, pad, c);
        account(t, c);
    }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < ECF8_NSYM; ++i) fold[wave][i] = tot[i];
    }
    __syncthreads();
    if (tid < ECF8_NSYM) {
        const uint64_t v = fold[0][tid] + fold[1][tid] + fold[2][tid] + fold[3][tid];
        if (v) atomicAdd(&freq[count_symbol(tid >> 1, tid & 1)], (unsigned long long)v);
    }
}

// Code bits of one tile from its counts.
__device__ __forceinline__ uint32_t tile_bits(const uint32_t* __restrict__ counts, uint64_t tile, const CountLens& L)
{
    const uint4 a = reinterpret_cast<const uint4*>(counts)[2 * tile];
    const uint4 b = reinterpret_cast<const uint4*>(counts)[2 * tile + 1];
    const uint32_t c[kCountWords] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t s = 0;
#pragma unroll
    for (int d = 0; d < kCountWords; ++d) s += (c[d] & 0xFFFFu) * L.v[2 * d] + (c[d] >> 16) * L.v[2 * d + 1];
    return s;
}

// Bits of the four tiles a scan lane owns (zero past the last tile).
__device__ __forceinline__ uint32_t lane_tiles(const uint32_t* __restrict__ counts, const CountLens& L, uint64_t tiles,
                                               uint64_t t0, uint32_t (&v)[4])
{
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[k] = t0 + k < tiles ? tile_bits(counts, t0 + k, L) : 0u;
        s += v[k];
    }
    return s;
}

// Inclusive scan over a workgroup of kLanes lanes (64-bit), `wsum` kLanes / 64 entries of LDS.
template <int kLanes>
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
    for (int w = 0; w < kLanes / 64; ++w) before += w < wave ? wsum[w] : 0ull;
    return v + before;
}

// x / d for x < 2^53 and 0 < d < 2^32: the rounded double quotient, corrected to the floor.
__device__ __forceinline__ uint64_t div_u64(uint64_t x, uint32_t d)
{
    uint64_t q = (uint64_t)((double)x / (double)d);
    if (q * d > x) --q;
    else if ((q + 1) * d <= x) ++q;
    return q;
}

// Pass 2a: total bits of each group of 1024 tiles.
__global__ __launch_bounds__(kScanLanes) void ecf8_group_sum_kernel(const uint32_t* __restrict__ counts, CountLens L,
                                                                    uint64_t tiles, uint64_t* __restrict__ gsum,
                                                                    EncTable tab, uint2* __restrict__ pairs)
{
    __shared__ uint64_t wsum[kScanLanes / 64];
    if (blockIdx.x == 0) {                                // the codeword-pair table (see lane_pairs)
        const uint32_t sa = threadIdx.x & 15u, sb = threadIdx.x >> 4;
        const uint32_t la = tab.len[sa], lb = tab.len[sb];
        pairs[threadIdx.x] = make_uint2((tab.code[sa] << lb) | tab.code[sb], la | ((la + lb) << 8));
    }
    uint32_t v[4];
    const uint64_t s = lane_tiles(counts, L, tiles, blockIdx.x * kGroupTiles + 4ull * threadIdx.x, v);
    const uint64_t incl = block_incl_scan<kScanLanes>(s, wsum);
    if (threadIdx.x == kScanLanes - 1) gsum[blockIdx.x] = incl;
}

// Pass 2b: tile bit offsets = the sum of the earlier groups' totals (each
// workgroup adds them up itself) + an exclusive scan inside the group
// (tile_off[tiles] = T), with the chunk and block holding each tile's first
// stream word.
__global__ __launch_bounds__(kScanLanes) void ecf8_tile_off_kernel(const uint32_t* __restrict__ counts, CountLens L,
                                                                   uint64_t tiles, const uint64_t* __restrict__ gsum,
                                                                   uint64_t* __restrict__ tile_off,
                                                                   uint64_t* __restrict__ tile_chunk, uint32_t chunk_bits,
                                                                   uint32_t tb)
{
    __shared__ uint64_t wsum[kScanLanes / 64];
    __shared__ uint64_t s_goff;
    // this group's offset: the earlier groups' totals, summed lane-strided
    uint64_t before = 0;
    for (uint64_t i = threadIdx.x; i < blockIdx.x; i += kScanLanes) before += gsum[i];
    before = block_incl_scan<kScanLanes>(before, wsum);
    if (threadIdx.x == kScanLanes - 1) s_goff = before;
    __syncthreads();
    const uint64_t goff = s_goff;
    uint32_t v[4];
    const uint64_t t0 = blockIdx.x * kGroupTiles + 4ull * threadIdx.x;
    const uint64_t s = lane_tiles(counts, L, tiles, t0, v);
    uint64_t run = goff + block_incl_scan<kScanLanes>(s, wsum) - s;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (t0 + k < tiles) {
            tile_off[t0 + k] = run;
            const uint64_t c = div_u64(run & ~31ull, chunk_bits);
            tile_chunk[2 * (t0 + k)] = c;
            tile_chunk[2 * (t0 + k) + 1] = div_u64(c, tb);
        }
        run += v[k];
        if (t0 + k + 1 == tiles) {
            tile_off[tiles] = run;
            const uint64_t c = div_u64(run & ~31ull, chunk_bits);
            tile_chunk[2 * tiles] = c;
            tile_chunk[2 * tiles + 1] = div_u64(c, tb);
        }
    }
}

// Inclusive scan over the 64 lanes of the wave: DPP row shifts inside each
// 16-lane row, then the earlier rows' totals through readlane.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane)
{
    v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 15);
    const uint32_t r1 = __builtin_amdgcn_readlane(v, 31);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane >> 4;
    return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// A tile's metadata, one 64-bit word per lane: lane 0 tile_off[tile], 1
// tile_off[tile + 1], 2..4 its chunk C0, block B0 and the next tile's chunk C1.
__device__ __forceinline__ uint64_t tile_meta(const EncArgs& a, uint64_t tile, int lane)
{
    if (lane >= 5) return 0;
    const uint64_t* p = lane < 2 ? a.tile_off + tile + lane : a.tile_chunk + 2 * tile + (lane - 2);
    return *p;
}

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// Nibble plane of one lane's 16 bytes: (s << 3) | m of each byte, element 0
// in the low nibble (SWAR: each byte's nibble, then two halvings).
__device__ __forceinline__ uint2 nibbles16(const uint32_t (&w)[4])
{
    uint32_t h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t x = ((w[q] >> 4) & 0x08080808u) | (w[q] & 0x07070707u);   // nibble in the low half of each byte
        x = (x | (x >> 4)) & 0x00FF00FFu;                                  // bytes 0 and 2: two nibbles each
        h[q] = (x | (x >> 8)) & 0xFFFFu;                                   // four nibbles, element 4q lowest
    }
    return make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
}

// Codeword pairs of one lane's 16 elements from the pair table `tbl`: entry
// s_a + 16 s_b holds pc = code(s_a) followed by code(s_b) (at most 32 bits)
// and pl = len(s_a) | (len(s_a) + len(s_b)) << 8.  The entry's byte offset
// 8 s_a + 128 s_b comes straight from the exponent bits (byte & 0x78 = 8 s).
// Elements at or past `valid` (ragged tail) get length 0.
template <bool kFull>
__device__ __forceinline__ void lane_pairs(const uint32_t (&w)[4], uint32_t valid, const uint2* tbl,
                                           uint32_t (&pc)[8], uint32_t (&pl)[8])
{
    const uint8_t* base = reinterpret_cast<const uint8_t*>(tbl);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t m = w[j >> 1] & 0x78787878u;
        const uint32_t ia = (m >> (16 * (j & 1))) & 0x78u, ib = (m >> (16 * (j & 1) + 8)) & 0x78u;
        const uint2 e = *reinterpret_cast<const uint2*>(base + ia + (ib << 4));
        pc[j] = e.x;
        pl[j] = e.y;
        if (!kFull) {
            if ((uint32_t)(2 * j) >= valid) {
                pc[j] = 0u;
                pl[j] = 0u;
            } else if ((uint32_t)(2 * j + 1) >= valid) {  // first codeword only
                pc[j] = e.x >> ((e.y >> 8) - (e.y & 255u));
                pl[j] = (e.y & 255u) * 257u;
            }
        }
    }
}

// Pass 3: encode, one workgroup per tile.
//   * The workgroup copies the pair table into LDS (one entry per lane).
//   * The tile's image words and gap words are cleared before the scan
//     barrier.
//   * A lane's 8 pairs are OR-ed into the LDS image at their bit positions,
//     each as a 64-bit window over two words.
//   * The chunk starts inside a lane's bit range (p, p + acc] are visited
//     one by one (most lanes have none): the pair holding one is found from
//     the cumulative pair ends E, its gap is the next codeword start after
//     it (the end of the pair's first codeword, or of the pair) minus the
//     chunk start, OR-ed into an LDS gap image (gap words from C0 / 8 on),
//     and a block start also stores the block offset.
//   * Chunk, block and position bookkeeping is 32-bit, relative to the
//     tile's chunk C0 and block B0.
__global__ __launch_bounds__(256) void ecf8_encode_kernel(EncArgs a)
{
    __shared__ uint32_t img[kTileWords];
    __shared__ uint32_t gimg[kGapWords];                  // gap words from word C0 / 8 on
    __shared__ uint32_t wsum[4];
    __shared__ uint2 s_pair[256];                         // the pair table
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t tile = blockIdx.x;
    const uint64_t e0 = tile * kTile + (uint64_t)tid * kEncPerLane;
    uint32_t w[4];
    load16(a.fp8, e0, a.n, w);
    const uint64_t tm = tile_meta(a, tile, lane);
    s_pair[tid] = a.pairs[tid];
    const uint64_t P0 = lane_u64(tm, 0), P1 = lane_u64(tm, 1), C0 = lane_u64(tm, 2), B0 = lane_u64(tm, 3),
                   C1 = lane_u64(tm, 4);
    const uint64_t W0 = P0 >> 5;                          // first stream word of the tile
    const uint64_t nw = P1 > P0 ? ((P1 + 31) >> 5) - W0 : 0;
    const uint32_t nwords = (uint32_t)(nw < (uint64_t)kTileWords - 1 ? nw : (uint64_t)kTileWords - 1);
    const uint32_t g_lo = (uint32_t)(((C0 + 1) >> 3) - (C0 >> 3));
    const uint64_t g_hi64 = C1 > C0 ? (C1 >> 3) - (C0 >> 3) + 1 : 0;
    const uint32_t g_hi = (uint32_t)(g_hi64 < (uint64_t)kGapWords ? g_hi64 : (uint64_t)kGapWords);
    for (uint32_t i = tid; i < nwords + 1; i += kEncLanes) img[i] = 0u;   // + 1: the last window's spill word
    for (uint32_t i = tid; i < g_hi; i += kEncLanes) gimg[i] = 0u;
    __syncthreads();                                      // pair table

    const uint32_t valid = e0 >= a.n ? 0u : (a.n - e0 >= (uint64_t)kEncPerLane ? 16u : (uint32_t)(a.n - e0));
    uint32_t pc[8], pl[8], E[8];
    if ((tile + 1) * kTile <= a.n)
        lane_pairs<true>(w, 16u, s_pair, pc, pl);
    else
        lane_pairs<false>(w, valid, s_pair, pc, pl);
    uint32_t acc = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        acc += pl[j] >> 8;
        E[j] = acc;                                       // end of pair j, from the lane's first bit
    }
    if (valid) *reinterpret_cast<uint2*>(a.nibbles + (e0 >> 1)) = nibbles16(w);

    const uint32_t incl = wave_incl_scan(acc, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();                                      // wsum; images cleared
    uint32_t before = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) before += v < wave ? wsum[v] : 0u;
    const uint32_t rel = (uint32_t)(P0 & 31) + before + incl - acc;   // bit offset inside the tile image

    // codeword pairs into the image: the pair's bits left-aligned in a 64-bit
    // window starting at its word (offset + length <= 63)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t pos = rel + (j ? E[j - 1] : 0u), L = pl[j] >> 8;
        const uint64_t v = (uint64_t)pc[j] << ((64u - (pos & 31u) - L) & 63u);
        atomicOr(&img[pos >> 5], (uint32_t)(v >> 32));
        atomicOr(&img[(pos >> 5) + 1], (uint32_t)v);
    }

    // chunk starts in (p, p + acc]: d = their offsets from the lane's first bit
    const uint32_t x = (uint32_t)((P0 & ~31ull) - C0 * a.chunk_bits) + rel;
    const uint32_t dt = div_small(x, a.m_chunk);
    uint32_t u = (uint32_t)(C0 & 7) + dt;                 // chunk of the lane's first bit - 8 * (C0 / 8)
    const uint32_t tbx = (uint32_t)(C0 - B0 * a.tb) + dt;
    uint32_t bk = div_small(tbx, a.m_tb);                 // its block - B0
    uint32_t tbp = tbx - bk * a.tb;                       // its place in the block
    for (uint32_t d = a.chunk_bits - (x - dt * a.chunk_bits); d <= acc; d += a.chunk_bits) {
        uint32_t st = 0, en = E[0], la = pl[0] & 255u, jj = 0;   // pair jj: E[jj - 1] < d <= E[jj]
#pragma unroll
        for (int k = 0; k < 7; ++k) {
            const bool past = E[k] < d;
            st = past ? E[k] : st;
            en = past ? E[k + 1] : en;
            la = past ? (pl[k + 1] & 255u) : la;
            jj += past ? 1u : 0u;
        }
        const uint32_t mid = st + la;                     // end of the pair's first codeword
        const bool in_a = d <= mid;
        const uint32_t gap = (in_a ? mid : en) - d;
        ++u;
        if (++tbp == a.tb) {
            tbp = 0;
            ++bk;
            const uint64_t blk = B0 + bk;
            if (blk <= a.n_blocks) a.blk_off[blk] = e0 + 2 * jj + (in_a ? 1 : 2);
        }
        if (gap && (u >> 3) < g_hi) atomicOr(&gimg[u >> 3], gap << (4 * (u & 7)));
    }
    __syncthreads();                                      // images complete

    // tile image -> stream (bytes MSB-first: each big-endian word
    // byte-swapped); words past the stream (metadata that undercounts T) are
    // dropped
    // A word the tile shares with its neighbour (the stream word holding a
    // tile boundary, the gap word holding chunks of both tiles) goes to the
    // tile's side slots instead; ecf8_boundary_kernel ORs the two tiles' parts
    // into it afterwards (global atomics here were 45% of the pass).  A tile
    // spans at least 4096 bits, so it shares a word with each neighbour at
    // most and no word has more than two tiles' bits.
    const bool last_tile = tile + 1 == a.tiles;
    const bool first_shared = (P0 & 31) != 0;
    const bool last_shared = (P1 & 31) != 0 && !last_tile;
    uint32_t* const side = a.side + 4 * tile;
    const uint32_t nout = W0 >= a.stream_words ? 0u
                          : (a.stream_words - W0 < (uint64_t)nwords ? (uint32_t)(a.stream_words - W0) : nwords);
    for (uint32_t i = tid; i < nout; i += kEncLanes) {
        const uint32_t v = __builtin_bswap32(img[i]);
        if (i == 0 && first_shared) side[0] = v;
        else if (i == nwords - 1 && last_shared) side[1] = v;
        else a.stream[W0 + i] = v;
    }
    // gap image -> gaps: the words of chunks C0 + 1 .. C1 (those starting in
    // (P0, P1]); the first is shared when chunk C0 (the previous tile's) is
    // in it, the last when chunk C1 + 1 (the next tile's) is
    const bool gfirst_shared = tile > 0 && ((C0 + 1) & 7) != 0;
    const bool glast_shared = !last_tile && (C1 & 7) != 7;
    for (uint32_t j = g_lo + tid; j < g_hi; j += kEncLanes) {
        const uint64_t g = (C0 >> 3) + j;
        if (g >= a.gap_words) break;
        const uint32_t v = gimg[j];
        if (j == g_lo && gfirst_shared) side[2] = v;
        else if (j + 1 == g_hi && glast_shared) side[3] = v;
        else a.gaps[g] = v;
    }
    // a tile with no chunk start (the last, if it is shorter than a chunk)
    // still shares the previous tile's gap word: its part is empty
    if (tid == 0 && g_lo >= g_hi) side[2] = 0u;
    if (last_tile) {                                      // zero padding after T
        for (uint64_t g = W0 + nwords + tid; g < a.stream_words; g += kEncLanes) a.stream[g] = 0u;
        // and the gap words past the tile's own (the last block's lanes that
        // hold no chunk; a tile with no chunk start wrote none: from the word
        // of chunk C0 + 1 on, which for tile 0 holds chunk 0)
        const uint64_t gz = C1 > C0 ? (C1 >> 3) + 1 : (C0 + 1) >> 3;
        for (uint64_t g = gz + tid; g < a.gap_words; g += kEncLanes) a.gaps[g] = 0u;
        if (tid == 0) {
            a.blk_off[0] = 0;
            a.blk_off[a.n_blocks] = a.n;
        }
    }
}

// Pass 4: the words two tiles share, one lane per tile boundary t (between
// tiles t and t + 1, at bit P = tile_off[t + 1]): the stream word holding P
// when P is not word-aligned, and the gap word holding chunks C1 = P / (8C)
// (tile t's last) and C1 + 1 (tile t + 1's first) when they share one.
__global__ __launch_bounds__(256) void ecf8_boundary_kernel(const uint64_t* __restrict__ tile_off, uint64_t tiles,
                                                            const uint32_t* __restrict__ side, uint32_t chunk_bits,
                                                            uint32_t* __restrict__ stream, uint64_t stream_words,
                                                            uint32_t* __restrict__ gaps, uint64_t gap_words)
{
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t + 1 >= tiles) return;
    const uint64_t P = tile_off[t + 1];
    const uint32_t* s0 = side + 4 * t;
    const uint32_t* s1 = side + 4 * (t + 1);
    if ((P & 31) != 0 && (P >> 5) < stream_words) stream[P >> 5] = s0[1] | s1[0];
    const uint64_t c1 = P / chunk_bits;
    if ((c1 & 7) != 7 && (c1 >> 3) < gap_words) gaps[c1 >> 3] = s0[3] | s1[2];
}

int check(hipError_t e) { return e == hipSuccess ? ECF8_OK : ECF8_ERR_HIP; }

// Workgroups of a 256-lane kernel resident on the current device at once
// (the grid of the persistent histogram kernel), per device and kernel.
std::mutex g_slots_mu;
std::vector<uint32_t> g_slots;

int resident_slots(int which, const void* kernel, uint32_t* out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ECF8_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_slots_mu);
    const size_t i = 2 * (size_t)dev + (size_t)which;
    if (g_slots.size() <= i) g_slots.resize(i + 1, 0u);
    if (!g_slots[i]) {
        int cus = 0, occ = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return ECF8_ERR_HIP;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 256, 0) != hipSuccess) return ECF8_ERR_HIP;
        g_slots[i] = (uint32_t)((cus > 0 ? cus : 1) * (occ > 0 ? occ : 1));
    }
    *out = g_slots[i];
    return ECF8_OK;
}

// Workspace: per-tile counts (32 B per tile) | tile bit offsets (tiles + 1,
// u64) | per-tile chunk and block (2 x u64) | group totals (u64) |
// codeword-pair table (2 KB) | per-tile side slots of the shared words
// (16 B per tile), each part 256-byte aligned.
struct EncWorkspace {
    uint64_t tiles, groups, off_off, chunk_off, group_off, pair_off, side_off, bytes;
};

EncWorkspace enc_workspace(uint64_t n)
{
    auto round = [](uint64_t x) { return (x + 255) / 256 * 256; };
    EncWorkspace w;
    w.tiles = (n + kTile - 1) / kTile;
    w.groups = (w.tiles + kGroupTiles - 1) / kGroupTiles;
    w.off_off = round(w.tiles * 4 * kCountWords);
    w.chunk_off = w.off_off + round((w.tiles + 1) * 8);
    w.group_off = w.chunk_off + round((w.tiles + 1) * 16);
    w.pair_off = w.group_off + round(w.groups * 8);
    w.side_off = w.pair_off + 256 * 8 + 256;
    w.bytes = w.side_off + round(w.tiles * 16);
    return w;
}

}  // namespace

extern "C" uint64_t ecf8_encode_workspace_bytes(uint64_t n)
{
    return enc_workspace(n).bytes;
}

extern "C" int ecf8_histogram_device(const uint8_t* fp8, uint64_t n, uint64_t* freq, void* workspace,
                                     uint64_t workspace_bytes, void* hip_stream)
{
    if ((!fp8 && n) || !freq || ((uintptr_t)freq & 7)) return ECF8_ERR_ARG;
    const EncWorkspace W = enc_workspace(n);
    if (workspace && (workspace_bytes < W.bytes || ((uintptr_t)workspace & 255))) return ECF8_ERR_WORKSPACE;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    hipLaunchKernelGGL(ecf8_zero_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<uint32_t*>(freq),
                       (uint64_t)2 * ECF8_NSYM);
    if (n) {
        uint32_t slots = 0;
        const int rc = resident_slots(0, reinterpret_cast<const void*>(ecf8_hist_kernel), &slots);
        if (rc) return rc;
        const uint64_t steps = (W.tiles + kHistWaves - 1) / kHistWaves;
        const uint64_t grid = steps < slots ? steps : slots;
        hipLaunchKernelGGL(ecf8_hist_kernel, dim3((uint32_t)grid), dim3(256), 0, st, fp8, n, W.tiles,
                           reinterpret_cast<unsigned long long*>(freq), reinterpret_cast<uint32_t*>(workspace));
    }
    return check(hipGetLastError());
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
    if (W.tiles > 0xFFFFFFFFull) return ECF8_ERR_SIZE;

    ecf8_codebook cb = meta->cb;
    uint32_t code[ECF8_NSYM];
    rc = ecf8_canonical_codes(&cb, code);
    if (rc) return rc;
    EncTable tab;
    for (int s = 0; s < ECF8_NSYM; ++s) {
        tab.code[s] = code[s];
        tab.len[s] = cb.len[s];
    }
    CountLens L;
    for (int d = 0; d < kCountWords; ++d)
        for (int f = 0; f < 2; ++f) L.v[2 * d + f] = cb.len[count_symbol(d, f)];
    uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
    const uint32_t* counts = reinterpret_cast<const uint32_t*>(ws);
    uint64_t* tile_off = reinterpret_cast<uint64_t*>(ws + W.off_off);
    uint64_t* tile_chunk = reinterpret_cast<uint64_t*>(ws + W.chunk_off);
    uint64_t* group = reinterpret_cast<uint64_t*>(ws + W.group_off);
    uint2* pairs = reinterpret_cast<uint2*>(ws + W.pair_off);
    uint32_t* side = reinterpret_cast<uint32_t*>(ws + W.side_off);
    EncArgs a;
    a.fp8 = fp8;
    a.n = n;
    a.tiles = W.tiles;
    a.n_blocks = meta->n_blocks;
    a.chunk_bits = 8u * meta->chunk_bytes;
    a.tb = meta->threads_per_block;
    a.gap_count = meta->n_blocks * meta->threads_per_block;
    a.gap_words = meta->gap_bytes / 4;
    a.stream_words = meta->stream_bytes / 4;   // C and TB are multiples of 4 and 64: a whole number of words
    a.stream = reinterpret_cast<uint32_t*>(stream);
    a.nibbles = nibbles;
    a.gaps = reinterpret_cast<uint32_t*>(gaps);
    a.blk_off = blk_off;
    a.tile_off = tile_off;
    a.tile_chunk = tile_chunk;
    a.pairs = pairs;
    a.side = side;
    a.m_chunk = ((1ull << 40) + a.chunk_bits - 1) / a.chunk_bits;
    a.m_tb = ((1ull << 40) + a.tb - 1) / a.tb;

    // every output word is written by the kernels: the gap and stream words a
    // tile owns by the encode kernel, those two tiles share by the boundary
    // kernel, the padding after the last chunk by the last tile
    hipLaunchKernelGGL(ecf8_group_sum_kernel, dim3((uint32_t)W.groups), dim3(kScanLanes), 0, st, counts, L, W.tiles,
                       group, tab, pairs);
    hipLaunchKernelGGL(ecf8_tile_off_kernel, dim3((uint32_t)W.groups), dim3(kScanLanes), 0, st, counts, L, W.tiles,
                       group, tile_off, tile_chunk, a.chunk_bits, a.tb);
    hipLaunchKernelGGL(ecf8_encode_kernel, dim3((uint32_t)W.tiles), dim3(kEncLanes), 0, st, a);
    if (W.tiles > 1)
        hipLaunchKernelGGL(ecf8_boundary_kernel, dim3((uint32_t)((W.tiles - 1 + 255) / 256)), dim3(256), 0, st,
                           tile_off, W.tiles, side, a.chunk_bits, a.stream, a.stream_words, a.gaps, a.gap_words);
    return check(hipGetLastError());
}
