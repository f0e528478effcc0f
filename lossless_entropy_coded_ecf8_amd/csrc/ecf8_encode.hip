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
// Two passes over the input:
//   1. histogram, in count tiles of 4096 elements: per tile, the count of
//      each of the 16 exponent symbols (kept in the workspace as 16-bit
//      fields) and the tensor's totals;
//   -- the host turns the totals into code lengths and sizes --
//   2. two small launches turn the per-tile counts and the code lengths into
//      64-bit tile bit offsets (tile bits = sum of count x length; group
//      totals over 1024 tiles, then each group adds up the totals before it
//      and scans its tiles) with the chunk and block of each tile's first
//      stream word, and write a 256-entry table of codeword pairs;
//   3. encode, one workgroup per 8192 elements (32 per lane): a lane looks up
//      its 16 element pairs in the pair table, lane and workgroup scans give
//      the bit positions, each pair is OR-ed into an LDS image of the
//      workgroup's bit range, and the image goes out in 16-byte stores; the
//      first and last stream word, when shared with a neighbouring
//      workgroup, go to side slots that a fourth launch ORs together.  Each
//      chunk start inside a lane's bit range gives that chunk's gap (next
//      codeword start - chunk start) into an LDS gap image, written out as
//      whole words (shared words through the side slots too), and a block
//      start the block offset; the nibble plane is written per lane.
//      Chunks are at least 32 bits and codewords at most 16, so an element's
//      bit interval holds at most one chunk start.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "ecf8.h"

namespace {

constexpr int kEncLanes = 256;
constexpr uint64_t kTile = 4096;                                       // elements per count tile
constexpr int kHistPerLane = 16;                                       // histogram: bytes per lane and load
constexpr int kEncPerLane = 32;                                        // encode: elements per lane
constexpr int kPairs = kEncPerLane / 2;                                // codeword pairs per lane
constexpr uint64_t kWgElems = (uint64_t)kEncLanes * kEncPerLane;       // 8192 elements per encode workgroup
constexpr uint64_t kWgTiles = kWgElems / kTile;                        // count tiles per encode workgroup
// LDS bit image of a workgroup's stream words: its bits (at most 16 per
// element), the offset of its first bit in a 16-byte aligned group of words
// (up to 3 words and 31 bits), the last window's spill word; whole quads.
constexpr int kImgWords = ((int)(kWgElems * ECF8_MAX_CODE_LEN / 32) + 1 + 3 + 1 + 3) / 4 * 4;
// LDS gap image: the bits span at most kImgWords * 32 bits, so (chunks being
// >= 32 bits) at most kImgWords + 1 chunk starts, 8 gaps per word; whole quads.
constexpr int kGapWords = ((kImgWords + 1) / 8 + 3 + 3) / 4 * 4;
constexpr int kScanLanes = 256;                                        // lanes of the per-group scans
constexpr uint64_t kGroupTiles = 4ull * kScanLanes;                    // tiles per scan group
constexpr int kCountWords = 8;                                         // per-tile counts: 16 x 16 bits
constexpr int kHistWaves = 4;                                          // histogram: one tile per wave at a time
constexpr int kHistLoads = (int)(kTile / 64 / kHistPerLane);           // 16-byte loads per lane per tile
static_assert(kWgElems % kTile == 0, "an encode workgroup covers whole count tiles");
constexpr uint64_t kMaxGrid = 1ull << 24;                              // workgroups of 256 lanes per launch

// Symbol counted by 16-bit field f (0 = low half) of per-tile count word d.
__host__ __device__ constexpr int count_symbol(int d, int f) { return (d >> 1) + 4 * (2 * (d & 1) + f); }

// One tensor of an encode launch: its input, outputs, workspace parts and
// code.  Up to kBatch tensors go to each launch by value (kernel argument).
struct EncJob {
    const uint8_t* fp8;
    uint64_t n;
    uint64_t tiles;            // count tiles: ceil(n / kTile)
    uint64_t n_wg;             // encode workgroups: ceil(n / kWgElems)
    uint64_t n_blocks;
    uint64_t gap_words;        // gap_bytes / 4
    uint64_t stream_words;     // stream_bytes / 4
    uint32_t* stream;
    uint8_t* nibbles;
    uint32_t* gaps;            // 4-byte words of the gap array
    uint64_t* blk_off;
    const uint32_t* counts;    // per-tile symbol counts (the histogram pass)
    uint64_t* group;           // per group of kGroupTiles tiles: its total bits
    uint64_t* tile_off;        // tiles + 1 entries; tile_off[tiles] = T
    uint64_t* tile_chunk;      // per tile and for T: chunk holding bit tile_off & ~31, and its block
    uint2* pairs;              // codeword-pair table, 256 entries
    uint32_t* side;            // per workgroup: its partial first and last stream words, first and last gap words
    uint64_t m_chunk;          // ceil(2^40 / chunk_bits)
    uint64_t m_tb;             // ceil(2^40 / tb)
    uint32_t chunk_bits;       // 8 * C
    uint32_t tb;               // chunks per block
    uint32_t stream_quads;     // stream is 16-byte aligned: whole quads of words go out as one store
    uint32_t nibble_quads;     // nibbles is 16-byte aligned
    uint16_t code[ECF8_NSYM];  // MSB-first canonical code per symbol
    uint8_t len[ECF8_NSYM];    // code length per symbol
    uint8_t count_len[2 * kCountWords];   // code length of the symbol of count field 2d + f
};

constexpr int kBatch = 8;

// The tensors of one launch and, per kernel, the first block of each tensor
// (start[count] = the grid).
struct EncBatch {
    EncJob job[kBatch];
    uint32_t grp_start[kBatch + 1];   // group-sum and tile-offset kernels
    uint32_t wg_start[kBatch + 1];    // encode kernel
    uint32_t bnd_start[kBatch + 1];   // boundary kernel
    uint32_t count;
};

// The tensor whose blocks hold block b (uniform): start[j] <= b < start[j + 1].
__device__ __forceinline__ int job_of(const uint32_t* start, uint32_t count, uint32_t b)
{
    int j = 0;
#pragma unroll
    for (int k = 1; k < kBatch; ++k) j += (k < (int)count && b >= start[k]) ? 1 : 0;
    return j;
}

// x / d for x < 2^20 and d <= 1024 through m = ceil(2^40 / d): the product's
// error is below x / 2^40 < 1 / d, so the quotient is exact.
__device__ __forceinline__ uint32_t div_small(uint32_t x, uint64_t m) { return (uint32_t)(((uint64_t)x * m) >> 40); }

// The lane's 16 bytes (elements e0 .. e0 + 15) as 4 little-endian words, zero past n.
__device__ __forceinline__ void load16(const uint8_t* p, uint64_t e0, uint64_t n, uint32_t (&w)[4])
{
    if (e0 + 16 <= n && ((uintptr_t)(p + e0) & 15) == 0) {
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
    const uint32_t lane_off = (uint32_t)lane * kHistPerLane;
    uint64_t t = first;
    uint4 nx[kHistLoads];
    auto load_full = [&](uint64_t tt) {
        const uint64_t s = tt < full ? tt : 0;            // past the last full tile: tile 0 again (discarded)
#pragma unroll
        for (int k = 0; k < kHistLoads; ++k)
            nx[k] = *reinterpret_cast<const uint4*>(fp8 + s * kTile + k * (64 * kHistPerLane) + lane_off);
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
            const uint64_t e0 = t * kTile + (uint64_t)k * (64 * kHistPerLane) + lane_off;
            load16(fp8, e0, n, w[k]);
            pad += e0 >= n ? kHistPerLane : (e0 + kHistPerLane > n ? (uint32_t)(e0 + kHistPerLane - n) : 0u);
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
__device__ __forceinline__ uint32_t tile_bits(const uint32_t* __restrict__ counts, uint64_t tile, const uint8_t* L)
{
    const uint4 a = reinterpret_cast<const uint4*>(counts)[2 * tile];
    const uint4 b = reinterpret_cast<const uint4*>(counts)[2 * tile + 1];
    const uint32_t c[kCountWords] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t s = 0;
#pragma unroll
    for (int d = 0; d < kCountWords; ++d) s += (c[d] & 0xFFFFu) * L[2 * d] + (c[d] >> 16) * L[2 * d + 1];
    return s;
}

// Bits of the four tiles a scan lane owns (zero past the last tile).
__device__ __forceinline__ uint32_t lane_tiles(const uint32_t* __restrict__ counts, const uint8_t* L, uint64_t tiles,
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

// Pass 2a: total bits of each group of 1024 tiles; the first group of each
// tensor also writes the tensor's codeword-pair table (see lane_pairs).
__global__ __launch_bounds__(kScanLanes) void ecf8_group_sum_kernel(const EncBatch B)
{
    __shared__ uint64_t wsum[kScanLanes / 64];
    const int jb = job_of(B.grp_start, B.count, blockIdx.x);
    const EncJob& J = B.job[jb];
    const uint32_t g = blockIdx.x - B.grp_start[jb];
    if (g == 0) {
        const uint32_t sa = threadIdx.x & 15u, sb = threadIdx.x >> 4;
        const uint32_t la = J.len[sa], lb = J.len[sb];
        const uint32_t pc = ((uint32_t)J.code[sa] << lb) | J.code[sb];    // la + lb <= 32 bits
        J.pairs[threadIdx.x] = make_uint2(la + lb ? pc << (32 - la - lb) : 0u, (la + lb) | (la << 16));
    }
    uint32_t v[4];
    const uint64_t s = lane_tiles(J.counts, J.count_len, J.tiles, g * kGroupTiles + 4ull * threadIdx.x, v);
    const uint64_t incl = block_incl_scan<kScanLanes>(s, wsum);
    if (threadIdx.x == kScanLanes - 1) J.group[g] = incl;
}

// Pass 2b: tile bit offsets = the sum of the earlier groups' totals (each
// workgroup adds them up itself) + an exclusive scan inside the group
// (tile_off[tiles] = T), with the chunk and block holding each tile's first
// stream word.
__global__ __launch_bounds__(kScanLanes) void ecf8_tile_off_kernel(const EncBatch B)
{
    __shared__ uint64_t wsum[kScanLanes / 64];
    __shared__ uint64_t s_goff;
    const int jb = job_of(B.grp_start, B.count, blockIdx.x);
    const EncJob& J = B.job[jb];
    const uint32_t g = blockIdx.x - B.grp_start[jb];
    const uint64_t tiles = J.tiles;
    // this group's offset: the earlier groups' totals, summed lane-strided
    uint64_t before = 0;
    for (uint64_t i = threadIdx.x; i < g; i += kScanLanes) before += J.group[i];
    before = block_incl_scan<kScanLanes>(before, wsum);
    if (threadIdx.x == kScanLanes - 1) s_goff = before;
    __syncthreads();
    const uint64_t goff = s_goff;
    uint32_t v[4];
    const uint64_t t0 = g * kGroupTiles + 4ull * threadIdx.x;
    const uint64_t s = lane_tiles(J.counts, J.count_len, tiles, t0, v);
    uint64_t run = goff + block_incl_scan<kScanLanes>(s, wsum) - s;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (t0 + k < tiles) {
            J.tile_off[t0 + k] = run;
            const uint64_t c = div_u64(run & ~31ull, J.chunk_bits);
            J.tile_chunk[2 * (t0 + k)] = c;
            J.tile_chunk[2 * (t0 + k) + 1] = div_u64(c, J.tb);
        }
        run += v[k];
        if (t0 + k + 1 == tiles) {
            J.tile_off[tiles] = run;
            const uint64_t c = div_u64(run & ~31ull, J.chunk_bits);
            J.tile_chunk[2 * tiles] = c;
            J.tile_chunk[2 * tiles + 1] = div_u64(c, J.tb);
        }
    }
}

// Inclusive scan over the 64 lanes of the wave: DPP row shifts inside each
// 16-lane row, then row_bcast:15 adds row r's total into row r + 1 and
// row_bcast:31 the first two rows' total into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v)
{
    v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return v;
}

// The lane's 32 bytes (elements e0 .. e0 + 31) as 8 little-endian words, zero past n.
__device__ __forceinline__ void load32(const uint8_t* p, uint64_t e0, uint64_t n, uint32_t (&w)[8])
{
    uint32_t a[4], b[4];
    load16(p, e0, n, a);
    load16(p, e0 + 16, n, b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        w[q] = a[q];
        w[4 + q] = b[q];
    }
}

// Nibble plane of 16 bytes: (s << 3) | m of each byte, element 0 in the low
// nibble.  Per word, a bit select (bitop3 with table 0xE4: the third operand
// picks the first where it is 1, else the second) puts the sign (bit 7,
// shifted to bit 3) beside the mantissa in each byte's low nibble (the high
// nibble is left dirty), a second select packs the low nibbles of bytes 2k
// and 2k + 1 into byte 2k, and a byte permute gathers bytes 0 and 2 of two
// words.
__device__ __forceinline__ uint32_t bit_select(uint32_t ones, uint32_t zeros, uint32_t mask)
{
    return __builtin_amdgcn_bitop3_b32(ones, zeros, mask, 0xE4);
}

__device__ __forceinline__ uint2 nibbles16(const uint32_t* w)
{
    uint32_t h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t x = bit_select(w[q], w[q] >> 4, 0x07070707u);   // low nibble: sign | mantissa
        h[q] = bit_select(x, x >> 4, 0x0F0F0F0Fu);                      // byte 2k: nibbles 2k, 2k + 1
    }
    return make_uint2(__builtin_amdgcn_perm(h[1], h[0], 0x06040200u), __builtin_amdgcn_perm(h[3], h[2], 0x06040200u));
}

// Codeword pairs of one lane's 32 elements from the pair table `tbl`: entry
// s_a + 16 s_b holds pc = code(s_a) followed by code(s_b), left-aligned in 32
// bits, and pl = (len(s_a) + len(s_b)) | len(s_a) << 16.  The entry's byte
// offset 8 s_a + 128 s_b comes straight from the exponent bits (byte & 0x78
// = 8 s).  Elements at or past `valid` (ragged tail) get length 0.
template <bool kFull>
__device__ __forceinline__ void lane_pairs(const uint32_t (&w)[8], uint32_t valid, const uint2* tbl,
                                           uint32_t (&pc)[kPairs], uint32_t (&pl)[kPairs])
{
    const uint8_t* base = reinterpret_cast<const uint8_t*>(tbl);
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
        const uint32_t h = w[j >> 1] >> (16 * (j & 1));
        const uint32_t off = (h & 0x78u) | ((h >> 4) & 0x780u);
        const uint2 e = *reinterpret_cast<const uint2*>(base + off);
        pc[j] = e.x;
        pl[j] = e.y;
        if (!kFull) {
            if ((uint32_t)(2 * j) >= valid) {
                pc[j] = 0u;
                pl[j] = 0u;
            } else if ((uint32_t)(2 * j + 1) >= valid) {  // first codeword only
                const uint32_t la = e.y >> 16;
                pc[j] = e.x & ~(0xFFFFFFFFu >> la);
                pl[j] = la * 0x10001u;
            }
        }
    }
}

// Pass 3: encode, one workgroup per 8192 elements (two count tiles), 32 per
// lane.
//   * The workgroup copies the pair table into LDS (one entry per lane); its
//     bit range, chunk and block come from the offsets of its first tile and
//     of the next workgroup's, read once (uniform).
//   * The bit image in LDS starts at the 16-byte aligned group of stream
//     words that holds the workgroup's first bit; it and the gap image are
//     cleared in quads before the scan barrier.
//   * A lane's 16 codeword pairs are OR-ed into the image at their bit
//     positions: the left-aligned pair shifted right by the position's offset
//     in its word, and the bits that spill into the next word (alignbit).
//   * The chunk starts inside a lane's bit range (p, p + acc] are visited one
//     by one (most lanes have none, a few one): the gap is the smallest
//     distance from the chunk start to a codeword start at or after it (the
//     starts of the pairs and of their second codewords, and the lane's end),
//     taken as a minimum of unsigned differences (starts before the chunk
//     wrap around to large values); it is OR-ed into the gap image (gap words
//     from C0 / 8 on), and a block start also stores the block offset: the
//     element whose codeword starts there, the count of codeword starts
//     before it.
//   * The image goes out in quads of words (one 16-byte store each; the
//     quads holding a word shared with a neighbouring workgroup word by word).
// Uniform state of one encode workgroup and its LDS.
struct WgState {
    uint64_t wg, e0, P0, P1, C0, B0, C1, W0, Wq;
    uint32_t o, nwords, g_lo, g_hi, valid;
    uint32_t* img;
    uint32_t* gimg;
    uint32_t* wsum;
    const uint2* pair;
};

// Everything after the pair-table barrier: kFull when all 8192 elements of
// the workgroup lie below n (no length-0 padding).
template <bool kFull>
__device__ __forceinline__ void encode_body(const EncJob& a, const WgState& S, const uint32_t (&w)[8])
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t pc[kPairs], pl[kPairs];
    lane_pairs<kFull>(w, S.valid, S.pair, pc, pl);
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < kPairs; ++j) sum += pl[j];
    const uint32_t acc = sum & 0xFFFFu;                   // the lane's bits (at most 512: no carry into bit 16)
    if (kFull || S.valid) {
        uint8_t* nib = a.nibbles + (S.e0 >> 1);
        const uint2 lo = nibbles16(w), hi = nibbles16(w + 4);
        if ((kFull || S.valid > 16) && a.nibble_quads) {
            *reinterpret_cast<uint4*>(nib) = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
            *reinterpret_cast<uint2*>(nib) = lo;
            if (kFull || S.valid > 16) *reinterpret_cast<uint2*>(nib + 8) = hi;
        }
    }

    const uint32_t incl = wave_incl_scan(acc);
    if (lane == 63) S.wsum[wave] = incl;
    __syncthreads();                                      // wsum; images cleared
    uint32_t before = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) before += v < wave ? S.wsum[v] : 0u;
    const uint32_t pre = before + incl - acc;             // the lane's first bit - P0
    const uint32_t ib = (uint32_t)(S.P0 & 127) + pre;     // ... in the image

    // codeword pairs into the image: bits [q, q + 32) of the pair at image
    // position q go to word q / 32 (shifted right by q % 32) and the next word
    // (the spill; zero when q % 32 = 0)
    uint32_t q[kPairs + 1];
    q[0] = ib;
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
        q[j + 1] = q[j] + (pl[j] & 0xFFFFu);
        atomicOr(&S.img[q[j] >> 5], pc[j] >> (q[j] & 31u));
        atomicOr(&S.img[(q[j] >> 5) + 1], __builtin_amdgcn_alignbit(pc[j], 0u, q[j]));
    }

    // chunk starts in (p, p + acc]: d = their offsets from the lane's first
    // bit, D = ib + d their image positions
    const uint32_t x = (uint32_t)(S.P0 - S.C0 * a.chunk_bits) + pre;   // from the start of chunk C0
    const uint32_t dt = div_small(x, a.m_chunk);
    uint32_t u = (uint32_t)(S.C0 & 7) + dt;               // chunk of the lane's first bit - 8 * (C0 / 8)
    const uint32_t tbx = (uint32_t)(S.C0 - S.B0 * a.tb) + dt;
    uint32_t bk = div_small(tbx, a.m_tb);                 // its block - B0
    uint32_t tbp = tbx - bk * a.tb;                       // its place in the block
    for (uint32_t d = a.chunk_bits - (x - dt * a.chunk_bits); d <= acc; d += a.chunk_bits) {
        uint32_t D = ib + d;
        asm volatile("" : "+v"(D));                       // one subtraction per codeword start and chunk start
        uint32_t gap = q[kPairs] - D;                     // the lane's end is the next lane's first start
#pragma unroll
        for (int j = 0; j < kPairs; ++j) {
            const uint32_t t = q[j] - D;                  // the pair's start; + len(s_a): its second codeword's
            gap = min(gap, min(t, t + (pl[j] >> 16)));
        }
        ++u;
        if (++tbp == a.tb) {
            tbp = 0;
            ++bk;
            const uint64_t blk = S.B0 + bk;
            if (blk <= a.n_blocks) {
                uint32_t before_d = 0;                    // codeword starts before the chunk start
#pragma unroll
                for (int j = 0; j < kPairs; ++j)
                    before_d += (q[j] < D ? 1u : 0u) + (q[j] + (pl[j] >> 16) < D ? 1u : 0u);
                asm volatile("" : "+v"(before_d));        // a 32-bit count, added to e0 once
                a.blk_off[blk] = S.e0 + before_d;
            }
        }
        if (gap && (u >> 3) < S.g_hi) atomicOr(&S.gimg[u >> 3], gap << (4 * (u & 7)));
    }
    __syncthreads();                                      // images complete

    // image -> stream (bytes MSB-first: each big-endian word byte-swapped);
    // words past the stream (metadata that undercounts T) are dropped.  A
    // word the workgroup shares with its neighbour (the stream word holding a
    // workgroup boundary, the gap word holding chunks of both) goes to the
    // workgroup's side slots instead; ecf8_boundary_kernel ORs the two parts
    // into it afterwards.  A workgroup other than the last spans at least
    // 8192 bits, so it shares a word with each neighbour at most and no word
    // has more than two workgroups' bits.
    const bool last_wg = S.wg + 1 == a.n_wg;
    const bool first_shared = (S.P0 & 31) != 0;
    const bool last_shared = (S.P1 & 31) != 0 && !last_wg;
    uint32_t* const side = a.side + 4 * S.wg;
    const uint32_t nwords = S.nwords, o = S.o;
    const uint32_t nout = S.W0 >= a.stream_words ? 0u
                          : (a.stream_words - S.W0 < (uint64_t)nwords ? (uint32_t)(a.stream_words - S.W0) : nwords);
    // image words [lo, hi) are the workgroup's own
    const uint32_t lo = o + (first_shared ? 1u : 0u);
    const uint32_t hi = o + (last_shared && nout == nwords ? nwords - 1 : nout);
    for (uint32_t k = tid; 4 * k < o + nout; k += kEncLanes) {
        const uint4 v = reinterpret_cast<const uint4*>(S.img)[k];
        const uint32_t val[4] = {__builtin_bswap32(v.x), __builtin_bswap32(v.y), __builtin_bswap32(v.z),
                                 __builtin_bswap32(v.w)};
        const uint32_t j0 = 4 * k;
        if (a.stream_quads && j0 >= lo && j0 + 4 <= hi) {
            *reinterpret_cast<uint4*>(a.stream + S.Wq + j0) = make_uint4(val[0], val[1], val[2], val[3]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t j = j0 + i;
                if (j >= lo && j < hi) a.stream[S.Wq + j] = val[i];
                else if (j == o && first_shared) side[0] = val[i];
                else if (j + 1 == o + nwords && last_shared && nout == nwords) side[1] = val[i];
            }
        }
    }
    // gap image -> gaps: the words of chunks C0 + 1 .. C1 (those starting in
    // (P0, P1]); the first is shared when chunk C0 (the previous workgroup's)
    // is in it, the last when chunk C1 + 1 (the next workgroup's) is
    const bool gfirst_shared = S.wg > 0 && ((S.C0 + 1) & 7) != 0;
    const bool glast_shared = !last_wg && (S.C1 & 7) != 7;
    for (uint32_t j = S.g_lo + tid; j < S.g_hi; j += kEncLanes) {
        const uint64_t g = (S.C0 >> 3) + j;
        if (g >= a.gap_words) break;
        const uint32_t v = S.gimg[j];
        if (j == S.g_lo && gfirst_shared) side[2] = v;
        else if (j + 1 == S.g_hi && glast_shared) side[3] = v;
        else a.gaps[g] = v;
    }
    // a workgroup with no chunk start (the last, if it is shorter than a
    // chunk) still shares the previous one's gap word: its part is empty
    if (tid == 0 && S.g_lo >= S.g_hi) side[2] = 0u;
    if (last_wg) {                                        // zero padding after T
        for (uint64_t g = S.W0 + nwords + tid; g < a.stream_words; g += kEncLanes) a.stream[g] = 0u;
        // and the gap words past the workgroup's own (the last block's lanes
        // that hold no chunk; a workgroup with no chunk start wrote none: from
        // the word of chunk C0 + 1 on, which for workgroup 0 holds chunk 0)
        const uint64_t gz = S.C1 > S.C0 ? (S.C1 >> 3) + 1 : (S.C0 + 1) >> 3;
        for (uint64_t g = gz + tid; g < a.gap_words; g += kEncLanes) a.gaps[g] = 0u;
        if (tid == 0) {
            a.blk_off[0] = 0;
            a.blk_off[a.n_blocks] = a.n;
        }
    }
}

// 7 workgroups per compute unit (72 VGPRs; 7 x 20.5 KB of LDS)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(7))) void ecf8_encode_kernel(const EncBatch B)
{
    __shared__ __align__(16) uint32_t img[kImgWords];
    __shared__ __align__(16) uint32_t gimg[kGapWords];     // gap words from word C0 / 8 on
    __shared__ uint32_t wsum[4];
    __shared__ uint2 s_pair[256];                         // the pair table
    const int tid = threadIdx.x;
    const int jb = job_of(B.wg_start, B.count, blockIdx.x);
    const EncJob& a = B.job[jb];
    WgState S;
    S.wg = blockIdx.x - B.wg_start[jb];
    const uint64_t t0 = S.wg * kWgTiles;
    const uint64_t t1 = t0 + kWgTiles < a.tiles ? t0 + kWgTiles : a.tiles;
    // uniform metadata: bit range [P0, P1), the chunk C0 and block B0 holding
    // word P0 / 32, the chunk C1 holding word P1 / 32
    S.P0 = a.tile_off[t0];
    S.P1 = a.tile_off[t1];
    S.C0 = a.tile_chunk[2 * t0];
    S.B0 = a.tile_chunk[2 * t0 + 1];
    S.C1 = a.tile_chunk[2 * t1];
    S.e0 = S.wg * kWgElems + (uint64_t)tid * kEncPerLane;
    uint32_t w[8];
    load32(a.fp8, S.e0, a.n, w);
    s_pair[tid] = a.pairs[tid];
    S.W0 = S.P0 >> 5;                                     // first stream word of the workgroup
    S.Wq = S.W0 & ~3ull;                                  // image word 0 = stream word Wq
    S.o = (uint32_t)(S.W0 - S.Wq);
    const uint64_t nw = S.P1 > S.P0 ? ((S.P1 + 31) >> 5) - S.W0 : 0;
    S.nwords = (uint32_t)(nw < (uint64_t)kImgWords - 8 ? nw : (uint64_t)kImgWords - 8);
    S.g_lo = (uint32_t)(((S.C0 + 1) >> 3) - (S.C0 >> 3));
    const uint64_t g_hi64 = S.C1 > S.C0 ? (S.C1 >> 3) - (S.C0 >> 3) + 1 : 0;
    S.g_hi = (uint32_t)(g_hi64 < (uint64_t)kGapWords ? g_hi64 : (uint64_t)kGapWords);
    S.valid = S.e0 >= a.n ? 0u : (a.n - S.e0 >= (uint64_t)kEncPerLane ? 32u : (uint32_t)(a.n - S.e0));
    S.img = img;
    S.gimg = gimg;
    S.wsum = wsum;
    S.pair = s_pair;
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    for (uint32_t k = tid; 4 * k < S.o + S.nwords + 1; k += kEncLanes) reinterpret_cast<uint4*>(img)[k] = z4;
    for (uint32_t k = tid; 4 * k < S.g_hi; k += kEncLanes) reinterpret_cast<uint4*>(gimg)[k] = z4;
    __syncthreads();                                      // pair table
    if ((S.wg + 1) * kWgElems <= a.n)
        encode_body<true>(a, S, w);
    else
        encode_body<false>(a, S, w);
}

// Pass 4: the words two workgroups share, one lane per boundary t (between
// workgroups t and t + 1, at bit P = tile_off[(t + 1) * kWgTiles]): the stream
// word holding P when P is not word-aligned, and the gap word holding chunks
// C1 = P / (8C) (workgroup t's last) and C1 + 1 (workgroup t + 1's first) when
// they share one.
__global__ __launch_bounds__(256) void ecf8_boundary_kernel(const EncBatch B)
{
    const int jb = job_of(B.bnd_start, B.count, blockIdx.x);
    const EncJob& J = B.job[jb];
    const uint64_t t = (uint64_t)(blockIdx.x - B.bnd_start[jb]) * blockDim.x + threadIdx.x;
    if (t + 1 >= J.n_wg) return;
    const uint64_t P = J.tile_off[(t + 1) * kWgTiles];
    const uint32_t* s0 = J.side + 4 * t;
    const uint32_t* s1 = J.side + 4 * (t + 1);
    if ((P & 31) != 0 && (P >> 5) < J.stream_words) J.stream[P >> 5] = s0[1] | s1[0];
    const uint64_t c1 = P / J.chunk_bits;
    if ((c1 & 7) != 7 && (c1 >> 3) < J.gap_words) J.gaps[c1 >> 3] = s0[3] | s1[2];
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
// codeword-pair table (2 KB) | per-encode-workgroup side slots of the shared words
// (16 B each, sized per tile), each part 256-byte aligned.
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

namespace {

// Checks one tensor's arguments and fills its job (n > 0), or sets `empty`
// (n = 0: the caller writes the 16 zero bytes of stream padding and
// blk_off[0] = 0).
int make_job(const ecf8_encode_job& in, EncJob& J, bool& empty)
{
    const ecf8_meta* meta = &in.meta;
    int rc = ecf8_validate_meta(meta);
    if (rc) return rc;
    const uint64_t n = meta->n;
    if (!in.stream || !in.blk_off || ((uintptr_t)in.stream & 3) || ((uintptr_t)in.blk_off & 7)) return ECF8_ERR_ARG;
    empty = n == 0;
    if (empty) return ECF8_OK;
    if (!in.fp8 || !in.nibbles || !in.gaps || !in.workspace || ((uintptr_t)in.nibbles & 7) ||
        ((uintptr_t)in.gaps & 3))
        return ECF8_ERR_ARG;
    const EncWorkspace W = enc_workspace(n);
    if (in.workspace_bytes < W.bytes || ((uintptr_t)in.workspace & 255)) return ECF8_ERR_WORKSPACE;
    const uint64_t n_wg = (n + kWgElems - 1) / kWgElems;
    if (n_wg >= kMaxGrid) return ECF8_ERR_SIZE;

    ecf8_codebook cb = meta->cb;
    uint32_t code[ECF8_NSYM];
    rc = ecf8_canonical_codes(&cb, code);
    if (rc) return rc;
    std::memset(&J, 0, sizeof(J));
    for (int s = 0; s < ECF8_NSYM; ++s) {
        J.code[s] = (uint16_t)code[s];
        J.len[s] = cb.len[s];
    }
    for (int d = 0; d < kCountWords; ++d)
        for (int f = 0; f < 2; ++f) J.count_len[2 * d + f] = cb.len[count_symbol(d, f)];
    uint8_t* ws = reinterpret_cast<uint8_t*>(in.workspace);
    J.fp8 = in.fp8;
    J.n = n;
    J.tiles = W.tiles;
    J.n_wg = n_wg;
    J.n_blocks = meta->n_blocks;
    J.gap_words = meta->gap_bytes / 4;
    J.stream_words = meta->stream_bytes / 4;   // C and TB are multiples of 4 and 64: a whole number of words
    J.stream = reinterpret_cast<uint32_t*>(in.stream);
    J.nibbles = in.nibbles;
    J.gaps = reinterpret_cast<uint32_t*>(in.gaps);
    J.blk_off = in.blk_off;
    J.counts = reinterpret_cast<const uint32_t*>(ws);
    J.group = reinterpret_cast<uint64_t*>(ws + W.group_off);
    J.tile_off = reinterpret_cast<uint64_t*>(ws + W.off_off);
    J.tile_chunk = reinterpret_cast<uint64_t*>(ws + W.chunk_off);
    J.pairs = reinterpret_cast<uint2*>(ws + W.pair_off);
    J.side = reinterpret_cast<uint32_t*>(ws + W.side_off);
    J.chunk_bits = 8u * meta->chunk_bytes;
    J.tb = meta->threads_per_block;
    J.m_chunk = ((1ull << 40) + J.chunk_bits - 1) / J.chunk_bits;
    J.m_tb = ((1ull << 40) + J.tb - 1) / J.tb;
    J.stream_quads = ((uintptr_t)in.stream & 15) == 0;
    J.nibble_quads = ((uintptr_t)in.nibbles & 15) == 0;
    return ECF8_OK;
}

// The four launches of up to kBatch tensors (every output word is written by
// them: the gap and stream words a workgroup owns by the encode kernel, those
// two workgroups share by the boundary kernel, the padding after the last
// chunk by the last workgroup).
int launch_batch(EncBatch& B, hipStream_t st)
{
    B.grp_start[0] = B.wg_start[0] = B.bnd_start[0] = 0;
    for (uint32_t j = 0; j < B.count; ++j) {
        const EncJob& J = B.job[j];
        B.grp_start[j + 1] = B.grp_start[j] + (uint32_t)((J.tiles + kGroupTiles - 1) / kGroupTiles);
        B.wg_start[j + 1] = B.wg_start[j] + (uint32_t)J.n_wg;
        B.bnd_start[j + 1] = B.bnd_start[j] + (uint32_t)((J.n_wg - 1 + 255) / 256);
    }
    for (uint32_t j = B.count + 1; j <= (uint32_t)kBatch; ++j)
        B.grp_start[j] = B.wg_start[j] = B.bnd_start[j] = 0xFFFFFFFFu;
    const uint32_t c = B.count;
    hipLaunchKernelGGL(ecf8_group_sum_kernel, dim3(B.grp_start[c]), dim3(kScanLanes), 0, st, B);
    hipLaunchKernelGGL(ecf8_tile_off_kernel, dim3(B.grp_start[c]), dim3(kScanLanes), 0, st, B);
    hipLaunchKernelGGL(ecf8_encode_kernel, dim3(B.wg_start[c]), dim3(kEncLanes), 0, st, B);
    if (B.bnd_start[c]) hipLaunchKernelGGL(ecf8_boundary_kernel, dim3(B.bnd_start[c]), dim3(256), 0, st, B);
    return check(hipGetLastError());
}

}  // namespace

extern "C" int ecf8_encode_batched_device(const ecf8_encode_job* jobs, int count, void* hip_stream)
{
    if (count < 0 || (count > 0 && !jobs)) return ECF8_ERR_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    std::vector<EncJob> J(count > 0 ? (size_t)count : 1);
    std::vector<char> empty(count > 0 ? (size_t)count : 1, 0);
    for (int i = 0; i < count; ++i) {           // every job checked before anything is launched
        bool e = false;
        const int rc = make_job(jobs[i], J[i], e);
        if (rc) return rc;
        empty[i] = e;
    }
    for (int i = 0; i < count; ++i) {
        if (!empty[i]) continue;
        hipLaunchKernelGGL(ecf8_zero_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<uint32_t*>(jobs[i].stream),
                           jobs[i].meta.stream_bytes / 4);
        hipLaunchKernelGGL(ecf8_zero_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<uint32_t*>(jobs[i].blk_off),
                           (uint64_t)2);
    }
    EncBatch B;
    B.count = 0;
    uint64_t wgs = 0;
    for (int i = 0; i <= count; ++i) {
        const bool flush = i == count || B.count == (uint32_t)kBatch || (!empty[i] && wgs + J[i].n_wg >= kMaxGrid);
        if (flush && B.count) {
            const int rc = launch_batch(B, st);
            if (rc) return rc;
            B.count = 0;
            wgs = 0;
        }
        if (i == count) break;
        if (empty[i]) continue;
        B.job[B.count++] = J[i];
        wgs += J[i].n_wg;
    }
    return check(hipGetLastError());
}

extern "C" int ecf8_encode_device(const uint8_t* fp8, const ecf8_meta* meta, uint8_t* stream, uint8_t* nibbles,
                                  uint8_t* gaps, uint64_t* blk_off, void* workspace, uint64_t workspace_bytes,
                                  void* hip_stream)
{
    if (!meta) return ECF8_ERR_ARG;
    ecf8_encode_job job;
    job.fp8 = fp8;
    job.meta = *meta;
    job.stream = stream;
    job.nibbles = nibbles;
    job.gaps = gaps;
    job.blk_off = blk_off;
    job.workspace = workspace;
    job.workspace_bytes = workspace_bytes;
    return ecf8_encode_batched_device(&job, 1, hip_stream);
}
