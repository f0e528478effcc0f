// ecf8v_decode.hip -- GPU decode of the BF16 (DFloat11 layout) and FP8 E5M2
// exponent-coding variants on MI355X (gfx950).  C ABI: include/ecf8v.h.
//
// Method: the DFloat11 article §3.2 (exponents decoded cooperatively inside a
// block, then the floats reassembled from exponent and the kept sign and
// mantissa) and §3.3 (a transformer block's tensors decoded together); the
// ECF8 technical blog §3.2.1 (each lane owns a chunk of the stream and starts
// at its stored gap, counts its codewords, a block-wide scan places them, the
// lanes decode into shared memory, the block writes back).
//
// Decode table (one per tensor, built on the GPU from the code lengths when
// the plan is prepared).  Canonical codes fill the 16-bit code space from 0
// in (length, symbol) order, so every codeword of at most 10 bits lies below
// every longer one:
//   * region 1: one entry per 10-bit prefix covered by codewords of at most
//     10 bits (p_long of them);
//   * region 2: one entry per 16-bit value of the space the longer codewords
//     take, then entries that decode nothing (unused code space, and padding
//     to at least 1025 entries and a multiple of 4).
// The index of a 32-bit window w is min(max(w >> 22, (w >> 16) - cdelta),
// last) with cdelta = 63 * p_long: one branch-free expression picks the
// region, and the clamp sends any window past the codes to an entry that
// decodes nothing.  As w >> 22 < 1024 <= last, the two bounds are one
// median-of-three.  When no code of a batch is longer than 10 bits there is no
// region 2 and the index is w >> 22 alone (the kernel's short form, chosen
// when the plan is prepared).  Codewords longer than 10 bits cover at most 1/8 of the
// space when there are at most 256 symbols, so a table has at most 9089
// entries.
// An entry holds the bits consumed (1 for no codeword), the whole codewords
// decoded (0..3), a no-codeword flag, and the symbols in bytes 1..3, first
// symbol lowest, bytes past the count zero.  BF16 symbols fill their bytes,
// so byte 0 holds the bits consumed (4..0), the count (6..5) and the flag
// (7).  E5M2 symbols sit in bits 6..2 of their bytes, where the output byte
// takes the exponent: byte 0 is the bits consumed alone (one byte-select
// subtract advances the walk), the count is in bits 9..8 and the flag in bit
// 15, around the first symbol (the write-back overwrites bits 7, 1 and 0 of
// every staged byte with the sign and mantissa).
//
// Decode kernel: persistent workgroups of TB lanes walk the global block
// index over all tensors; each block's stream chunks, gaps and offsets are
// loaded one block ahead.  Per block:
//   * the lanes' 16-byte chunks plus a look-ahead word go to LDS in
//     word-major rows, so a 32-bit window at any bit position is two LDS
//     reads and a funnel shift;
//   * counting walk: lookups in wave-uniform steps of four, each entry
//     recorded in statically indexed registers (lanes past their chunk end
//     record 0; an E5M2 wave whose chunks are all whole takes its first two
//     steps without that test); a lane's last lookup may decode codewords
//     starting past its chunk, which are taken off its count;
//   * block scan of the counts (checked against the block offsets);
//   * replay: each recorded entry's symbol bytes are OR-ed into the cleared
//     LDS stage at the scanned position (one dword OR per entry; the part
//     that crosses into the next dword is carried to the next entry's OR).  Codewords a lane
//     decodes past its chunk end are the next lane's first ones, at the same
//     positions, so OR-ing them twice is exact.  Lanes with more lookups than
//     records walk the rest from registers;
//   * write back in units of 16 output bytes (8 BF16 or 16 E5M2 elements):
//     the unit's staged symbols and its 8 raw-plane bytes make its elements
//     with byte permutes and masks, one non-temporal 16-byte buffer store per
//     unit, so a wave's store covers 1 KB of contiguous output; the ragged
//     ends element by element from the same assembled words.  Every raw group a lane writes is loaded during
//     the replay, and the next block's inputs are taken before the stores are
//     issued, so no load waits behind the stores.  The lane that reads a
//     group clears it for the next block.
// Blocks of more than 16384 symbols (codes averaging under 2 bits) take a
// slower path: rounds of 16384 symbols, each lane walking its chunk again.
// Wave priority rises through a block (walk 1, scan and replay 2, write-back
// 3), so the wave of a SIMD nearest its stores issues first.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "ecf8v.h"

namespace {

constexpr int kChunk = 16;                  // bytes per lane
constexpr int kChunkBits = 8 * kChunk;
constexpr int kWin = 10;                    // region-1 window bits
constexpr int kLongShift = 16 - kWin;
constexpr int kTabMax = 9092;               // entries per table (at most 9089 used), a multiple of 4
constexpr int kTabMin = 1028;               // 1025 rounded up to a multiple of 4
constexpr int kStageSyms = 16384;           // symbols staged per block on the fast path
constexpr int kStageBytes = kStageSyms + 64;   // + alignment shift, symbols OR-ed past the end
constexpr int kRecords = 20;                // table entries recorded per lane by the counting walk
constexpr int kStep = 4;                    // lookups per wave-uniform step of the walk
// Write-back unit: the elements of 16 output bytes, 8 (BF16) or 16 (E5M2),
// with 8 bytes of raw plane either way; one 16-byte store per unit, so that a
// wave's store covers 1 KB of contiguous output.
template <int kFmt>
struct Unit {
    static constexpr uint32_t kElems = kFmt == ECF8V_BF16 ? 8u : 16u;
    static constexpr int kPerLane = kFmt == ECF8V_BF16 ? 8 : 4;   // loaded per lane after the block scan:
                                                                  // with 256 lanes, all of a fast-path block
};
constexpr int kRawMax = 8;                  // the larger of the two kPerLane
constexpr int kTableSlices = (kTabMax + 255) / 256;

// Entry fields per format (see the table description above).
template <int kFmt>
struct Entry {
    static constexpr uint32_t kNb = kFmt == ECF8V_BF16 ? 31u : 255u;       // bits consumed: e & kNb
    static constexpr int kCnt = kFmt == ECF8V_BF16 ? 5 : 8;               // codewords: (e >> kCnt) & 3
    static constexpr uint32_t kInv = kFmt == ECF8V_BF16 ? 0x80u : 0x8000u;   // no codeword
    static constexpr int kSymShift = kFmt == ECF8V_BF16 ? 0 : 2;          // symbol i: (e >> (8 + 8 i + kSymShift))
    static constexpr uint32_t kSym = kFmt == ECF8V_BF16 ? 255u : 31u;     //   & kSym
};
static_assert(kRecords % kStep == 0 && kStep % 2 == 0, "records are taken kStep at a time, looked up in pairs");
constexpr int kSureSteps = (kChunkBits / 16) / kStep;   // steps whose lookups all start inside a whole chunk
static_assert(kSureSteps * kStep <= kRecords && 15 + 16 * (kSureSteps * kStep - 1) < kChunkBits, "sure steps");

// Per-tensor descriptor in the workspace.
struct DescV {
    const uint8_t* stream;
    const uint8_t* raw;
    const uint8_t* gaps;
    const uint64_t* blk_off;
    uint8_t* out;
    uint64_t n;
    uint64_t first_block;      // global index of the tensor's first block
    uint64_t end_block;        // one past its last
    uint64_t total_bits;       // T: codewords start only before it
    int32_t cdelta;            // 63 * p_long
    uint32_t p_long;           // 10-bit prefixes covered by codewords of at most 10 bits
    uint32_t long_units;       // 16-bit code values taken by the longer codewords
    uint32_t entries;          // table entries (the last decodes nothing), a multiple of 4
    uint8_t len[ECF8V_MAX_SYM];
};

// Workspace: status (bad-block counter) | descriptors | one table per tensor,
// each part 256-byte aligned.
constexpr uint64_t kStatusBytes = 256;
uint64_t desc_offset() { return kStatusBytes; }
uint64_t table_offset(int count) { return desc_offset() + ((uint64_t)count * sizeof(DescV) + 255) / 256 * 256; }

// Table geometry of a code (host): region sizes and the entry count.
struct TabGeo {
    uint32_t p_long, long_units, entries;
    int32_t cdelta;
};

TabGeo table_geometry(const uint8_t* len)
{
    uint32_t short_units = 0, all_units = 0;
    for (int s = 0; s < ECF8V_MAX_SYM; ++s) {
        if (!len[s]) continue;
        const uint32_t u = 1u << (16 - len[s]);
        all_units += u;
        if (len[s] <= kWin) short_units += u;
    }
    TabGeo g;
    g.p_long = short_units >> kLongShift;
    g.long_units = all_units - short_units;
    g.cdelta = (int32_t)(g.p_long * ((1u << kLongShift) - 1));
    uint32_t e = g.p_long + g.long_units + 1;
    if (e < (uint32_t)kTabMin) e = kTabMin;
    g.entries = (e + 3) & ~3u;
    return g;
}

// ------------------------------------------------------------ memory helpers

// Global memory through an address-space-1 pointer (the descriptor pointers
// are generic; generic accesses also count against the LDS/scalar wait counter).
#define ECF8V_GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 gld16(const void* p)
{
    const ECF8V_GLOBAL u32x4* q = (const ECF8V_GLOBAL u32x4*)p;
    const u32x4 v = *q;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Buffer resources for the streaming loads and stores: wave-uniform base and
// byte size, 32-bit lane offsets, hardware range checks (loads past the end
// read 0, stores past the end are dropped).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;      // raw, untyped dword access
constexpr int kNonTemporal = 2;             // cache-policy bit: output stores and raw-plane loads (used once)
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint64_t bytes)
{
    const uint32_t nr = bytes < 0xFFFFFFFFull ? (uint32_t)bytes : 0xFFFFFFFFu;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nr, kRsrcWord3);
}
__device__ __forceinline__ uint32_t bld1(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0); }
__device__ __forceinline__ uint32_t bld(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
template <int kPolicy = 0>
__device__ __forceinline__ uint2 bld2_p(Rsrc r, uint32_t off, uint32_t soff)
{
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, kPolicy);
    return make_uint2(v.x, v.y);
}
template <int kPolicy = 0>
__device__ __forceinline__ uint4 bld4_p(Rsrc r, uint32_t off, uint32_t soff)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kPolicy);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 bld2(Rsrc r, uint32_t off, uint32_t soff = 0) { return bld2_p<0>(r, off, soff); }
__device__ __forceinline__ uint4 bld4(Rsrc r, uint32_t off, uint32_t soff = 0) { return bld4_p<0>(r, off, soff); }
__device__ __forceinline__ void bst4(Rsrc r, uint32_t off, uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    u32x4 v;
    v.x = a;
    v.y = b;
    v.z = c;
    v.w = d;
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kNonTemporal);
}
__device__ __forceinline__ void bst2(Rsrc r, uint32_t off, uint16_t v) { __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0); }
__device__ __forceinline__ void bst1(Rsrc r, uint32_t off, uint8_t v) { __builtin_amdgcn_raw_buffer_store_b8(v, r, off, 0, 0); }

__device__ __forceinline__ uint32_t bswap(uint32_t x) { return __builtin_bswap32(x); }

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// ------------------------------------------------------------ table kernel
// Grid (tensors, kTableSlices) of 256 lanes: workgroup (i, j) builds entries
// [256 j, 256 j + 256) of tensor i's table, one entry per lane.  Lane s first
// places symbol s in canonical order (its rank and the left-justified start
// of its code range); an entry is then decoded greedily from its known bits
// (10 in region 1, 16 in region 2) by binary search over the code starts.
__global__ __launch_bounds__(256) void ecf8v_table_kernel(const DescV* __restrict__ descs, uint32_t* __restrict__ tables,
                                                          uint32_t fmt)
{
    __shared__ uint32_t s_start[ECF8V_MAX_SYM];
    __shared__ uint8_t s_len[ECF8V_MAX_SYM];
    __shared__ uint8_t s_sym[ECF8V_MAX_SYM];
    __shared__ uint32_t s_k;
    const DescV& d = descs[blockIdx.x];
    const int tid = threadIdx.x;
    const uint32_t entries = d.entries;
    if (blockIdx.y * 256u >= entries) return;                 // uniform per workgroup
    if (tid == 0) s_k = 0;
    __syncthreads();
    const uint32_t l = d.len[tid];
    if (l) {
        uint32_t rank = 0, start = 0;
        for (int u = 0; u < ECF8V_MAX_SYM; ++u) {
            const uint32_t lu = d.len[u];
            if (lu && (lu < l || (lu == l && u < tid))) {
                ++rank;
                start += 1u << (16 - lu);
            }
        }
        s_start[rank] = start;
        s_len[rank] = (uint8_t)l;
        s_sym[rank] = (uint8_t)tid;
        atomicAdd(&s_k, 1u);
    }
    __syncthreads();
    const int k = (int)s_k;
    const uint32_t idx = blockIdx.y * 256u + tid;
    if (idx >= entries) return;
    uint32_t v = 0, known = 0;
    if (idx < d.p_long) {
        v = idx << kLongShift;
        known = kWin;
    } else if (idx < d.p_long + d.long_units) {
        v = idx + (uint32_t)d.cdelta;
        known = 16;
    }
    uint32_t pos = 0, ns = 0, sy = 0;
    while (k > 0 && ns < 3 && pos < known) {
        const uint32_t x = (v << pos) & 0xFFFFu;
        int lo = 0, hi = k;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_start[mid] <= x) lo = mid;
            else hi = mid;
        }
        const uint32_t ll = s_len[lo];
        if (x < s_start[lo] || x - s_start[lo] >= (1u << (16 - ll))) break;   // unused code space
        if (pos + ll > known) break;                                         // codeword not fully known
        sy |= (uint32_t)s_sym[lo] << (8 * ns);
        ++ns;
        pos += ll;
    }
    const bool bf = fmt == ECF8V_BF16;
    const uint32_t cnt_shift = bf ? (uint32_t)Entry<ECF8V_BF16>::kCnt : (uint32_t)Entry<ECF8V_E5M2>::kCnt;
    const uint32_t sym_shift = bf ? (uint32_t)Entry<ECF8V_BF16>::kSymShift : (uint32_t)Entry<ECF8V_E5M2>::kSymShift;
    const uint32_t inv = 1u | (bf ? Entry<ECF8V_BF16>::kInv : Entry<ECF8V_E5M2>::kInv);
    tables[(uint64_t)blockIdx.x * kTabMax + idx] = ns ? (pos | (ns << cnt_shift) | (sy << (8 + sym_shift))) : inv;
}

__global__ __launch_bounds__(64) void ecf8v_clear_kernel(unsigned long long* status, uint32_t words)
{
    if (threadIdx.x < words) status[threadIdx.x] = 0ull;
}

// ------------------------------------------------------------ decode helpers

// Block inputs loaded one block ahead: the lane's chunk, the look-ahead word,
// the byte holding its gap, and (lanes 0 and 1) the block's two offsets.
struct BlockIn {
    uint4 sv;
    uint32_t la;
    uint32_t gb;
    uint64_t off;
};

// Descriptor fields the prefetch needs, cached per tensor.
struct NextTensor {
    int t;
    uint64_t begin, end, n;
    const uint8_t* stream;
    const uint8_t* gaps;
    const uint64_t* blk_off;
};

__device__ __forceinline__ void fetch_tensor(const DescV* descs, int t, NextTensor& nt)
{
    const DescV* d = descs + t;
    nt.t = t;
    nt.begin = d->first_block;
    nt.end = d->end_block;
    nt.n = d->n;
    nt.stream = d->stream;
    nt.gaps = d->gaps;
    nt.blk_off = d->blk_off;
}

template <int kTB>
__device__ __forceinline__ void load_block(const NextTensor& nt, uint64_t gblk, int tid, BlockIn& in)
{
    const uint64_t b = gblk - nt.begin;
    const uint2 o = bld2(make_rsrc(nt.blk_off + b, 16), (tid & 1) * 8u);
    in.off = ((uint64_t)o.y << 32) | o.x;
    // the stream has 16 bytes past its last block for the last look-ahead
    const Rsrc rs = make_rsrc(nt.stream + b * (kTB * kChunk), kTB * kChunk + 16);
    in.sv = bld4(rs, tid * kChunk);
    in.la = bld(rs, tid * kChunk + kChunk);
    in.gb = bld1(make_rsrc(nt.gaps + b * (kTB / 2), kTB / 2), tid >> 1);
}

// Output range of a block (or round): elements [lo, lo + nw), units of
// `unit` elements counted from base = lo rounded down to a unit (a0 = lo - base).
struct BlockGeo {
    uint64_t lo, base, want;
    uint32_t nw, a0, units;
    bool sane;          // lo <= hi <= n
};

__device__ __forceinline__ BlockGeo block_geo(uint64_t lo_raw, uint64_t hi_raw, uint64_t n, uint32_t unit)
{
    BlockGeo g;
    g.sane = lo_raw <= hi_raw && hi_raw <= n;
    const uint64_t hi = hi_raw < n ? hi_raw : n;
    g.lo = lo_raw < hi ? lo_raw : hi;
    g.want = hi - g.lo;
    g.nw = g.want < (uint64_t)kStageSyms ? (uint32_t)g.want : (uint32_t)kStageSyms;
    g.base = g.lo & ~(uint64_t)(unit - 1);
    g.a0 = (uint32_t)(g.lo - g.base);
    g.units = (g.a0 + g.nw + unit - 1) / unit;
    return g;
}

// The raw plane of the units of a range, 8 bytes per unit (the resource ends
// with the range, so loads past it read 0 without touching memory).
template <int kFmt>
__device__ __forceinline__ Rsrc raw_rsrc(const uint8_t* raw, const BlockGeo& g)
{
    return make_rsrc(raw + (kFmt == ECF8V_BF16 ? g.base : g.base >> 1), 8ull * g.units);
}

// Output elements from base on, to the end of the tensor.
template <int kFmt>
__device__ __forceinline__ Rsrc out_rsrc(uint8_t* out, uint64_t base, uint64_t n)
{
    const uint64_t eb = kFmt == ECF8V_BF16 ? 2 : 1;
    return make_rsrc(out + eb * base, eb * (n - base));
}

__device__ __forceinline__ uint2 load_raw_unit(Rsrc rr, uint32_t u) { return bld2(rr, 8u * u); }

// The symbols of a unit as staged: 8 bytes (BF16) or 16 (E5M2).
template <int kFmt>
__device__ __forceinline__ uint4 read_unit(const uint8_t* stage, uint32_t u)
{
    if constexpr (kFmt == ECF8V_BF16) {
        const uint2 v = reinterpret_cast<const uint2*>(stage)[u];
        return make_uint4(v.x, v.y, 0u, 0u);
    } else {
        return reinterpret_cast<const uint4*>(stage)[u];
    }
}
template <int kFmt>
__device__ __forceinline__ void clear_unit(uint8_t* stage, uint32_t u)
{
    if constexpr (kFmt == ECF8V_BF16)
        reinterpret_cast<uint2*>(stage)[u] = make_uint2(0u, 0u);
    else
        reinterpret_cast<uint4*>(stage)[u] = make_uint4(0u, 0u, 0u, 0u);
}

// Bit-field insert: the bits of a where m is set, of b elsewhere.  One
// three-input bitwise instruction (truth table 0xca: m ? a : b); written as
// (a & m) | (b & ~m) the compiler splits it into masks and ORs.
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b)
{
    return __builtin_amdgcn_bitop3_b32(m, a, b, 0xca);
}

// The elements of a unit from its staged symbols and its raw plane, as the 4
// words of its 16 output bytes: byte permutes, shifts and bit-field inserts.
template <int kFmt>
__device__ __forceinline__ void assemble_unit(uint4 sv, uint2 rv, uint32_t (&o)[4])
{
    if constexpr (kFmt == ECF8V_BF16) {
        // element = raw bit 7 (sign) << 15 | exponent << 7 | raw bits 6..0
        const uint32_t S[2] = {sv.x, sv.y}, R[2] = {rv.x, rv.y};
#pragma unroll
        for (int q = 0; q < 4; ++q) {                     // elements 2q, 2q + 1 into word q
            const uint32_t rr = __builtin_amdgcn_perm(0u, R[q >> 1], (q & 1) ? 0x03030202u : 0x01010000u);
            const uint32_t ss = __builtin_amdgcn_perm(0u, S[q >> 1], (q & 1) ? 0x0c030c02u : 0x0c010c00u);
            o[q] = bfi(0x807F807Fu, rr, ss << 7);         // each half: raw byte twice | exponent byte at bit 7
        }
    } else {
        // element = nibble bit 2 (sign) << 7 | exponent << 2 | nibble bits 1..0;
        // the staged bytes hold the exponent in bits 6..2 already (bits 7, 1,
        // 0 may carry entry flags: the two inserts overwrite them)
        const uint32_t S[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {                     // elements 4q .. 4q + 3 into word q
            const uint32_t y = __builtin_amdgcn_perm(0u, q < 2 ? rv.x : rv.y, (q & 1) ? 0x03030202u : 0x01010000u);
            const uint32_t t = bfi(0x00FF00FFu, y, y >> 4);   // nibble j in bits 3..0 of byte j
            o[q] = bfi(0x80808080u, t << 5, bfi(0x03030303u, t, S[q]));
        }
    }
}

// A whole unit: one 16-byte store.
template <int kFmt>
__device__ __forceinline__ void write_unit(Rsrc ro, uint32_t u, uint4 sv, uint2 rv)
{
    uint32_t o[4];
    assemble_unit<kFmt>(sv, rv, o);
    bst4(ro, 16u * u, o[0], o[1], o[2], o[3]);
}

// A ragged unit ue of a range (range-relative elements [a0, endo)): the unit
// is assembled whole, its elements inside the range stored one by one.
template <int kFmt>
__device__ __forceinline__ void write_edge(Rsrc ro, uint32_t ue, uint4 sv, uint2 rv, uint32_t a0, uint32_t endo)
{
    constexpr uint32_t kE = Unit<kFmt>::kElems;
    uint32_t o[4];
    assemble_unit<kFmt>(sv, rv, o);
#pragma unroll
    for (uint32_t e = 0; e < kE; ++e) {
        const uint32_t i = kE * ue + e;
        if (i >= a0 && i < endo) {
            if constexpr (kFmt == ECF8V_BF16)
                bst2(ro, 2u * i, (uint16_t)(o[e >> 1] >> (16 * (e & 1))));
            else
                bst1(ro, i, (uint8_t)(o[e >> 2] >> (8 * (e & 3))));
        }
    }
}

// Write back a range: range-relative elements [a0, endo), element i staged
// at stage[i].  Lane tid writes the whole units u = tid + k * kTB with one
// 16-byte store each, the first kPre of them with the raw plane already in
// rv; lane 0 writes a ragged first unit (its raw plane rv[0] when kPre > 0)
// and lane end_full % kTB a ragged last unit (its raw plane tail_raw when
// kPre > 0) element-wise.  The lane that reads a unit from the stage clears it.
template <int kFmt, int kTB, int kPre>
__device__ __forceinline__ void write_back(uint8_t* stage, Rsrc rr, Rsrc ro, uint32_t a0, uint32_t endo, int tid,
                                           const uint2 (&rv)[kRawMax], uint2 tail_raw)
{
    constexpr uint32_t kE = Unit<kFmt>::kElems;
    const uint32_t first_full = a0 ? 1u : 0u;
    const uint32_t end_full = endo / kE;                 // units [first_full, end_full) are whole
    const uint32_t units = (endo + kE - 1) / kE;
    uint32_t u = (uint32_t)tid;
#pragma unroll
    for (int k = 0; k < kPre; ++k, u += kTB) {
        // E5M2 runs 7 waves per SIMD (72 registers): the unit indices are
        // recomputed per block rather than kept across it, where the register
        // allocator would put them in scratch
        if constexpr (kFmt == ECF8V_E5M2) asm volatile("" : "+v"(u));
        if (u >= first_full && u < end_full) {
            const uint4 sv = read_unit<kFmt>(stage, u);
            clear_unit<kFmt>(stage, u);
            write_unit<kFmt>(ro, u, sv, rv[k]);
        }
    }
    for (; u < end_full; u += kTB) {
        if (u >= first_full) {
            const uint4 sv = read_unit<kFmt>(stage, u);
            clear_unit<kFmt>(stage, u);
            write_unit<kFmt>(ro, u, sv, load_raw_unit(rr, u));
        }
    }
    if (a0 && tid == 0) {                                // unit 0 (which may also be the last)
        const uint4 sv = read_unit<kFmt>(stage, 0u);
        clear_unit<kFmt>(stage, 0u);
        write_edge<kFmt>(ro, 0u, sv, kPre > 0 ? rv[0] : load_raw_unit(rr, 0u), a0, endo);
    }
    if (end_full < units && end_full >= first_full && (uint32_t)tid == end_full % kTB) {
        const uint4 sv = read_unit<kFmt>(stage, end_full);
        clear_unit<kFmt>(stage, end_full);
        write_edge<kFmt>(ro, end_full, sv, kPre > 0 ? tail_raw : load_raw_unit(rr, end_full), a0, endo);
    }
}

// OR the symbol bytes of an entry into the stage at byte position ob (its
// 24 bits straddle at most two dwords).
__device__ __forceinline__ void emit_entry(uint32_t* stage32, uint32_t ob, uint32_t e)
{
    const uint64_t v = (uint64_t)(e >> 8) << (8 * (ob & 3));
    uint32_t* w = stage32 + (ob >> 2);
    atomicOr(w, (uint32_t)v);
    atomicOr(w + 1, (uint32_t)(v >> 32));
}

// The same for consecutive entries of a lane, one LDS atomic each: the
// entry's bytes cover dword ob / 4 and, when they cross, part of the next.
// Only the first is OR-ed here, together with `carry`, the previous entry's
// spill into this same dword; this entry's spill is returned in `carry` for
// the next entry (or the final flush).  An entry adds at most 3 bytes, so the
// next one starts in this dword or the next, and a spill is non-zero only if
// it starts in the next: the carry lands in the dword it belongs to.
__device__ __forceinline__ void emit_entry_carry(uint32_t* stage32, uint32_t ob, uint32_t e, uint32_t& carry)
{
    const uint64_t v = (uint64_t)(e >> 8) << (8 * (ob & 3));
    atomicOr(stage32 + (ob >> 2), (uint32_t)v | carry);
    carry = (uint32_t)(v >> 32);
}

// Window at chunk bit p from the lane's words in registers (w[4] the look-ahead).
__device__ __forceinline__ uint32_t reg_window(const uint32_t (&w)[5], uint32_t p)
{
    const uint32_t k = p >> 5;
    uint32_t hi = w[0], lo = w[1];
    if (k == 1) { hi = w[1]; lo = w[2]; }
    if (k == 2) { hi = w[2]; lo = w[3]; }
    if (k >= 3) { hi = w[3]; lo = w[4]; }
    return (uint32_t)(((((uint64_t)hi << 32) | lo) << (p & 31)) >> 32);
}

// min(max(a, b), last) for a = win >> 22 <= 1023 < last: the median of the
// three (one instruction).  kShort: every code of the batch is at most 10
// bits long (no region 2), so a is the index itself: one shift.  (With an
// incomplete code the prefixes past the codes are entries that decode
// nothing in either form.)
template <bool kShort>
__device__ __forceinline__ uint32_t tab_index(uint32_t win, int cd, int last)
{
    int a = (int)(win >> (32 - kWin));
    if (kShort) {
        // kept opaque, so that the entry's address is one shift-and-add of it
        // (not a shift, a mask and an add of the window)
        asm volatile("" : "+v"(a));
        return (uint32_t)a;
    }
    const int b = (int)(win >> 16) - cd;
    int m;
    asm("v_med3_i32 %0, %1, %2, %3" : "=v"(m) : "v"(b), "v"(a), "s"(last));
    return (uint32_t)m;
}


// Waves per SIMD the register allocation must allow (measured best with 256
// lanes: BF16 keeps its 16 raw-plane registers per lane unspilled at 5 (at 6
// a record spills), E5M2 fits 7); smaller workgroups are held lower by the
// stage's LDS (16 KB per workgroup of any size, 160 KB per compute unit of 4
// SIMDs).
template <int kFmt, int kTB>
constexpr int kMinWaves = (kFmt == ECF8V_BF16 ? 5 : 7) < (160 * 1024 / (kStageBytes + 64)) * (kTB / 64) / 4
                              ? (kFmt == ECF8V_BF16 ? 5 : 7)
                              : (160 * 1024 / (kStageBytes + 64)) * (kTB / 64) / 4;

// Static LDS: the stage (the stream rows live inside it) at address 0, so a
// row address is a lane offset OR-ed with a row offset; then the wave sums.
// Dynamic LDS: code lengths (256 bytes) | table (tab_n entries).
template <int kWaves>
struct StageLds {
    uint8_t stage[kStageBytes];
    uint32_t wsum[kWaves];
};
template <int kFmt, int kTB, bool kShort>
__global__ __launch_bounds__(kTB) __attribute__((amdgpu_waves_per_eu(kMinWaves<kFmt, kTB>))) void ecf8v_decode_kernel(
    const DescV* __restrict__ descs, int count, const uint32_t* __restrict__ tables, uint64_t total_blocks,
    unsigned long long* __restrict__ status, uint32_t tab_n)
{
    constexpr int kWaves = kTB / 64;
    constexpr uint32_t kPitch = 4u * kTB;                      // bytes per row
    constexpr int kPitchShift = kTB == 256 ? 5 : (kTB == 128 ? 4 : 3);   // (r & 0xE0) << s == (r >> 5) * kPitch
    static_assert(7 * kPitch <= (uint32_t)kStageBytes, "rows inside the stage");
    constexpr uint32_t kE = Unit<kFmt>::kElems;
    using En = Entry<kFmt>;
    __shared__ __align__(16) StageLds<kWaves> s_lds;
    extern __shared__ __align__(16) uint8_t dyn[];
    uint8_t* const stage = s_lds.stage;
    uint32_t* const stage32 = reinterpret_cast<uint32_t*>(s_lds.stage);
    uint32_t* const s_wsum = s_lds.wsum;
    uint8_t* const s_len = dyn;
    uint32_t* const s_tab = reinterpret_cast<uint32_t*>(dyn + ECF8V_MAX_SYM);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // Row rho (0..5) sits at stage + kPitch * (rho + 1), lane tid's dword at
    // + 4 tid; word w of the lane's chunk (w = 4: look-ahead) in row 4 - w,
    // row 5 only feeds a window's discarded half.  With r = 160 - p for chunk
    // bit p, the window at p is alignbit(row (r >> 5), row (r >> 5) - 1, r);
    // a lane past its end may read row -1 (stage bytes [0, kPitch)).
    uint32_t* const col = reinterpret_cast<uint32_t*>(stage + kPitch) + tid;
    const uint32_t col_lo = (uint32_t)tid * 4u;

    uint64_t blk = blockIdx.x;
    if (blk >= total_blocks) return;
    for (int i = tid; i < kStageBytes / 16; i += kTB) reinterpret_cast<uint4*>(stage)[i] = make_uint4(0u, 0u, 0u, 0u);

    NextTensor nt;
    fetch_tensor(descs, 0, nt);
    while (nt.t + 1 < count && blk >= nt.end) fetch_tensor(descs, nt.t + 1, nt);
    BlockIn nx;
    load_block<kTB>(nt, blk, tid, nx);
    int ptens = nt.t;
    // the first block's inputs are taken here, so that at the loop head only
    // the back edge has loads in flight (whose order the compiler then knows)
    asm volatile("" ::"v"(nx.sv.x), "v"(nx.la), "v"(nx.gb), "v"((uint32_t)nx.off));

    int cur = -1;
    uint64_t c_begin = 0, c_n = 0, c_T = 0;
    const uint8_t* c_raw = nullptr;
    const uint8_t* c_stream = nullptr;
    uint8_t* c_out = nullptr;
    int c_cd = 0, c_last = 0;

    for (; blk < total_blocks; blk += gridDim.x) {
        const BlockIn in = nx;
        uint2 rc[kRawMax];
        if (ptens != cur) {
            // every lane is past the previous block's last table read
            const DescV* d = descs + ptens;
            c_begin = d->first_block;
            c_n = d->n;
            c_T = d->total_bits;
            c_raw = d->raw;
            c_stream = d->stream;
            c_out = d->out;
            c_cd = d->cdelta;
            const uint32_t ne = d->entries <= tab_n ? d->entries : tab_n;
            c_last = (int)ne - 1;
            const uint32_t* tx = tables + (uint64_t)ptens * kTabMax;
            // the lane index passes through an empty asm so that the per-lane
            // addresses of these copies are formed here, when a tensor
            // changes, instead of being hoisted out of the block loop and
            // kept live (at 7 waves per SIMD they would be spilled)
            int lt = tid;
            asm volatile("" : "+v"(lt));
            for (uint32_t i = lt; i < ne / 4; i += kTB) reinterpret_cast<uint4*>(s_tab)[i] = gld16(tx + 4 * i);
            for (int i = lt; i < ECF8V_MAX_SYM; i += kTB) s_len[i] = d->len[i];
            cur = ptens;
        }
        // the table is in place and the previous block's write-back (which
        // clears the stage memory the rows reuse) is done
        __syncthreads();
        col[4 * kTB] = bswap(in.sv.x);
        col[3 * kTB] = bswap(in.sv.y);
        col[2 * kTB] = bswap(in.sv.z);
        col[1 * kTB] = bswap(in.sv.w);
        col[0] = bswap(in.la);
        const uint64_t b = blk - c_begin;
        const uint64_t cstart = (b * kTB + tid) * (uint64_t)kChunkBits;
        const uint32_t E = c_T > cstart ? (c_T - cstart < (uint64_t)kChunkBits ? (uint32_t)(c_T - cstart) : (uint32_t)kChunkBits) : 0u;
        const uint32_t gap = (in.gb >> ((tid & 1) * 4)) & 15u;
        const BlockGeo geo = block_geo(lane_u64(in.off, 0), lane_u64(in.off, 1), c_n, kE);

        // prefetch the next block of this workgroup (after the last block the
        // current one is loaded again: unconditional loads keep the wait counts exact)
        const uint64_t nb = blk + gridDim.x;
        const uint64_t nbe = nb < total_blocks ? nb : blk;
        while (nt.t + 1 < count && nbe >= nt.end) fetch_tensor(descs, nt.t + 1, nt);
        load_block<kTB>(nt, nbe, tid, nx);
        ptens = nt.t;

        // Wave priorities rise through the block: walk 1, scan and replay 2,
        // write-back 3, then 0 until the next walk, so the wave of a SIMD
        // nearest its stores issues first.
        __builtin_amdgcn_s_setprio(1);
        // ---- counting walk, recording each lookup's entry
        const int cd = c_cd, last = c_last;
        const uint32_t rend = 160u - E;
        const uint32_t r0 = 160u - gap;
        uint32_t rec[kRecords];
        uint32_t r = r0, cnt = 0, inv = 0, lastex = 0;
        bool act = r > rend;
        int nq = 0;                           // four-lookup steps taken (wave-uniform)
        // An E5M2 wave whose 64 chunks all lie below T takes its first
        // kSureSteps steps without activity tests: a lookup consumes at most
        // 16 bits and the walk starts at most 15 bits in, so each of the first
        // 8 lookups starts inside the 128-bit chunk.  (BF16 keeps one path:
        // at 5 waves per SIMD the second one would spill records.)
        constexpr int kSure = kFmt == ECF8V_E5M2 ? kSureSteps : 0;
        const bool wave_full =
            c_T >= (b * kTB + (uint64_t)((__builtin_amdgcn_readfirstlane(tid) & ~63) + 64)) * (uint64_t)kChunkBits;
#pragma unroll
        for (int q = 0; q < kRecords / kStep; ++q) {
            // lookups in pairs: the second takes the first's window shifted by
            // the bits the first consumed (at most 16, so the 16 bits an index
            // reads are still stream bits); its rows are not read again
            if (q < kSure && wave_full) {
                nq = q + 1;
                uint32_t win = 0;
#pragma unroll
                for (int j = 0; j < kStep; ++j) {
                    if (j % 2 == 0) {
                        const uint32_t a = col_lo | ((r & 0xE0u) << kPitchShift);   // col_lo < kPitch
                        const uint32_t wlo = *reinterpret_cast<const uint32_t*>(stage + a);
                        const uint32_t whi = *reinterpret_cast<const uint32_t*>(stage + a + kPitch);
                        win = __builtin_amdgcn_alignbit(whi, wlo, r);
                    } else {
                        win <<= rec[kStep * q + j - 1] & En::kNb & 31u;
                    }
                    const uint32_t e = s_tab[tab_index<kShort>(win, cd, last)];
                    rec[kStep * q + j] = e;
                    r -= e & En::kNb;
                    cnt += (e >> En::kCnt) & 3u;
                    if (j % 2) inv |= rec[kStep * q + j - 1] | e;
                }
                lastex = rec[kStep * q + kStep - 1];
                act = r > rend;
                continue;
            }
            if (__builtin_amdgcn_ballot_w64(act) == 0) break;
            nq = q + 1;
            uint32_t win = 0;
#pragma unroll
            for (int j = 0; j < kStep; ++j) {
                if (j % 2 == 0) {
                    const uint32_t a = col_lo | ((r & 0xE0u) << kPitchShift);   // col_lo < kPitch
                    const uint32_t wlo = *reinterpret_cast<const uint32_t*>(stage + a);
                    const uint32_t whi = *reinterpret_cast<const uint32_t*>(stage + a + kPitch);
                    win = __builtin_amdgcn_alignbit(whi, wlo, r);
                } else {
                    win <<= rec[kStep * q + j - 1] & En::kNb & 31u;
                }
                const uint32_t e = s_tab[tab_index<kShort>(win, cd, last)];
                const uint32_t em = act ? e : 0u;
                rec[kStep * q + j] = em;
                lastex = act ? e : lastex;
                r -= em & En::kNb;
                cnt += (em >> En::kCnt) & 3u;
                if (j % 2) inv |= rec[kStep * q + j - 1] | em;
                act = r > rend;
            }
        }
        const uint32_t r_rec = r;            // where the recorded lookups end
        while (r > rend) {
            const uint32_t a = col_lo | ((r & 0xE0u) << kPitchShift);
            const uint32_t wlo = *reinterpret_cast<const uint32_t*>(stage + a);
            const uint32_t whi = *reinterpret_cast<const uint32_t*>(stage + a + kPitch);
            const uint32_t e = s_tab[tab_index<kShort>(__builtin_amdgcn_alignbit(whi, wlo, r), cd, last)];
            lastex = e;
            r -= e & En::kNb;
            cnt += (e >> En::kCnt) & 3u;
            inv |= e;
        }
        __builtin_amdgcn_s_setprio(2);
        // the lane's rows are stage memory from here on: leave them cleared
#pragma unroll
        for (int k = 0; k < 5; ++k) col[k * kTB] = 0u;
        if (r != r0) {
            // the last lookup started `room` bits before the chunk end: keep
            // its codewords that start before it
            const uint32_t ns = (lastex >> En::kCnt) & 3u;
            const uint32_t room = r + (lastex & En::kNb) - rend;
            const uint32_t l1 = s_len[(lastex >> (8 + En::kSymShift)) & En::kSym];
            const uint32_t l2 = s_len[(lastex >> (16 + En::kSymShift)) & En::kSym];
            const uint32_t keep = 1u + (ns >= 2 && l1 < room ? 1u : 0u) + (ns >= 3 && l1 + l2 < room ? 1u : 0u);
            cnt -= ns - keep;
        }
        // a window with no codeword spoils the block's total
        if (inv & En::kInv) cnt += 1u << 22;

        // ---- block scan of the counts
        uint32_t x = cnt;
        x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);
        x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);
        x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);
        x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);
        const uint32_t q0 = __builtin_amdgcn_readlane(x, 15), q1 = __builtin_amdgcn_readlane(x, 31),
                       q2 = __builtin_amdgcn_readlane(x, 47), q3 = __builtin_amdgcn_readlane(x, 63);
        const int row = lane >> 4;
        x += (row >= 1 ? q0 : 0u) + (row >= 2 ? q1 : 0u) + (row >= 3 ? q2 : 0u);
        if (lane == 0) s_wsum[__builtin_amdgcn_readfirstlane(tid) >> 6] = q0 + q1 + q2 + q3;   // this wave's
        __syncthreads();
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t sw = s_wsum[w];
            before += w < wave ? sw : 0u;
            total += sw;
        }
        const uint32_t pos = before + x - cnt;
        const bool ok = geo.sane && total == geo.want;

        // the next block's inputs have been in flight during the walk: take
        // them into registers now, before this block's stores are issued (a
        // later wait for them would also wait for those stores)
        asm volatile("" ::"v"(nx.sv.x), "v"(nx.sv.y), "v"(nx.sv.z), "v"(nx.sv.w), "v"(nx.la), "v"(nx.gb),
                     "v"((uint32_t)nx.off), "v"((uint32_t)(nx.off >> 32)));
        if (ok && total <= (uint32_t)kStageSyms) {
            // the block's raw plane, in flight during the replay (loaded a
            // block ahead instead, it measured slower: more registers live
            // across the walk, and the loads queued behind the stores)
            const Rsrc rr = raw_rsrc<kFmt>(c_raw, geo);
#pragma unroll
            for (int k = 0; k < Unit<kFmt>::kPerLane; ++k)   // read once: non-temporal
                rc[k] = bld2_p<kNonTemporal>(rr, 8u * tid, 8u * k * kTB);
            // and the ragged last unit's, for the lane that writes it (other
            // lanes load past the range: no memory access)
            const uint32_t endo = geo.a0 + geo.nw, end_full = endo / kE;
            const bool tail_lane = (endo % kE) && end_full >= (geo.a0 ? 1u : 0u) && (uint32_t)tid == end_full % kTB;
            const uint2 tail_raw = load_raw_unit(rr, tail_lane ? end_full : 0x0FFFFFFFu);
            // ---- replay into the stage
            uint32_t ob = geo.a0 + pos;
            uint32_t carry = 0;
#pragma unroll
            for (int q = 0; q < kRecords / kStep; ++q) {
                if (q < nq) {                             // no early exit: the records keep static indices
#pragma unroll
                    for (int j = 0; j < kStep; ++j) {
                        const uint32_t e = rec[kStep * q + j];
                        emit_entry_carry(stage32, ob, e, carry);
                        ob += (e >> En::kCnt) & 3u;
                    }
                }
            }
            // the last entry's spill belongs to ob's dword (zero if it did not cross)
            if (nq) atomicOr(stage32 + (ob >> 2), carry);
            if (r_rec > rend) {
                // lanes with more lookups than records: the rest from registers
                // (the rows are stage memory now; the chunk is L2-resident)
                const Rsrc rs = make_rsrc(c_stream + b * (kTB * kChunk), kTB * kChunk + 16);
                const uint4 cv = bld4(rs, tid * kChunk);
                const uint32_t w[5] = {bswap(cv.x), bswap(cv.y), bswap(cv.z), bswap(cv.w),
                                       bswap(bld(rs, tid * kChunk + kChunk))};
                uint32_t r2 = r_rec;
                while (r2 > rend) {
                    const uint32_t e = s_tab[tab_index<kShort>(reg_window(w, 160u - r2), cd, last)];
                    emit_entry(stage32, ob, e);
                    ob += (e >> En::kCnt) & 3u;
                    r2 -= e & En::kNb;
                }
            }
            __syncthreads();
            __builtin_amdgcn_s_setprio(3);
            // ---- write back; every unit read is cleared
            write_back<kFmt, kTB, Unit<kFmt>::kPerLane>(stage, rr, out_rsrc<kFmt>(c_out, geo.base, c_n), geo.a0, endo,
                                                        tid, rc, tail_raw);
            __builtin_amdgcn_s_setprio(0);
            // symbols OR-ed past the block's end (by the last lane, or decoded
            // from the padding after T) lie in the units up to zend
            const uint32_t zend0 = (geo.a0 + total + 2u + 16u) / kE;
            const uint32_t zend = zend0 < (uint32_t)kStageBytes / kE ? zend0 : (uint32_t)kStageBytes / kE;
            for (uint32_t u = geo.units + tid; u < zend; u += kTB) clear_unit<kFmt>(stage, u);
        } else if (ok) {
            // ---- more than kStageSyms symbols: rounds, each lane walking its
            // chunk again and writing its symbols of the round
            const Rsrc rs = make_rsrc(c_stream + b * (kTB * kChunk), kTB * kChunk + 16);
            const uint4 cv = bld4(rs, tid * kChunk);
            const uint32_t w[5] = {bswap(cv.x), bswap(cv.y), bswap(cv.z), bswap(cv.w),
                                   bswap(bld(rs, tid * kChunk + kChunk))};
            for (uint32_t base = 0; base < total; base += kStageSyms) {
                const uint32_t lim = total - base < (uint32_t)kStageSyms ? total - base : (uint32_t)kStageSyms;
                const uint64_t j_start = geo.lo + base;
                const uint32_t shift = (uint32_t)(j_start & (kE - 1));
                if (pos < base + lim && pos + cnt > base) {
                    uint32_t p = gap, k = pos;
                    while (p < E && k < base + lim) {
                        const uint32_t e = s_tab[tab_index<kShort>(reg_window(w, p), cd, last)];
                        const uint32_t ns = (e >> En::kCnt) & 3u;
                        for (uint32_t i = 0; i < ns; ++i, ++k)
                            if (k >= base && k < base + lim && k < pos + cnt)
                                stage[k - base + shift] = (uint8_t)(e >> (8 + 8 * i));
                        p += e & En::kNb;
                    }
                }
                __syncthreads();
                const BlockGeo rg = block_geo(j_start, j_start + lim, c_n, kE);
                write_back<kFmt, kTB, 0>(stage, raw_rsrc<kFmt>(c_raw, rg), out_rsrc<kFmt>(c_out, rg.base, c_n), rg.a0,
                                         rg.a0 + rg.nw, tid, rc, rc[0]);
                __syncthreads();
            }
        } else if (tid == 0) {
            atomicAdd(status, 1ull);
        }
    }
}

int check(hipError_t e) { return e == hipSuccess ? ECF8_OK : ECF8_ERR_HIP; }

template <int kFmt, int kTB>
const void* decode_kernel_ptr(bool short_codes)
{
    return short_codes ? reinterpret_cast<const void*>(ecf8v_decode_kernel<kFmt, kTB, true>)
                       : reinterpret_cast<const void*>(ecf8v_decode_kernel<kFmt, kTB, false>);
}

const void* pick_kernel(uint32_t fmt, uint32_t tb, bool short_codes)
{
    if (fmt == ECF8V_BF16) {
        if (tb == 64) return decode_kernel_ptr<ECF8V_BF16, 64>(short_codes);
        if (tb == 128) return decode_kernel_ptr<ECF8V_BF16, 128>(short_codes);
        if (tb == 256) return decode_kernel_ptr<ECF8V_BF16, 256>(short_codes);
    } else if (fmt == ECF8V_E5M2) {
        if (tb == 64) return decode_kernel_ptr<ECF8V_E5M2, 64>(short_codes);
        if (tb == 128) return decode_kernel_ptr<ECF8V_E5M2, 128>(short_codes);
        if (tb == 256) return decode_kernel_ptr<ECF8V_E5M2, 256>(short_codes);
    }
    return nullptr;
}

std::mutex g_mu;
std::map<std::tuple<int, uint32_t, uint32_t, uint32_t, bool>, uint32_t> g_slots;   // (device, fmt, tb, lds, form)

// Resident decode workgroups of the current device for a kernel and its dynamic LDS.
int kernel_slots(uint32_t fmt, uint32_t tb, uint32_t lds, bool short_codes, uint32_t* out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ECF8_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    const auto key = std::make_tuple(dev, fmt, tb, lds, short_codes);
    auto it = g_slots.find(key);
    if (it == g_slots.end()) {
        int cus = 0, occ = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return ECF8_ERR_HIP;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, pick_kernel(fmt, tb, short_codes), (int)tb, lds) !=
            hipSuccess)
            return ECF8_ERR_HIP;
        it = g_slots.emplace(key, (uint32_t)((cus > 0 ? cus : 1) * (occ > 0 ? occ : 1))).first;
    }
    *out = it->second;
    return ECF8_OK;
}

uint32_t decode_lds_bytes(uint32_t tab_n) { return (uint32_t)ECF8V_MAX_SYM + 4 * tab_n; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" uint64_t ecf8v_workspace_bytes(int count)
{
    if (count < 0) return 0;
    return table_offset(count) + (uint64_t)count * kTabMax * 4;
}

extern "C" int ecf8v_decode_prepare(const ecf8v_tensor_desc* descs, int count, uint8_t* out_base, void* workspace,
                                    uint64_t workspace_bytes, void* hip_stream, ecf8v_plan* plan)
{
    if (!plan || count < 0 || (count > 0 && (!descs || !out_base))) return ECF8_ERR_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < ecf8v_workspace_bytes(count))
        return ECF8_ERR_WORKSPACE;
    std::memset(plan, 0, sizeof(*plan));
    std::vector<DescV> dv(count);
    uint64_t blocks = 0;
    uint32_t tab_n = kTabMin;
    uint32_t fmt = count ? descs[0].meta.format : ECF8V_BF16, tb = count ? descs[0].meta.threads_per_block : 256;
    bool short_codes = true;              // no codeword longer than 10 bits in any tensor: the one-shift index
    for (int i = 0; i < count; ++i) {
        const ecf8v_tensor_desc& t = descs[i];
        int rc = ecf8v_validate_meta(&t.meta);
        if (rc) return rc;
        if (t.meta.format != fmt || t.meta.threads_per_block != tb) return ECF8_ERR_ARG;
        if (t.meta.chunk_bytes != (uint32_t)kChunk || !pick_kernel(fmt, tb, false)) return ECF8_ERR_UNSUPPORTED;
        if (t.meta.n && (!t.stream || !t.raw || !t.gaps || !t.blk_off)) return ECF8_ERR_ARG;
        if (!aligned(t.stream, 16) || !aligned(t.blk_off, 8) || (t.out_offset & 15) ||
            !aligned(t.raw, fmt == ECF8V_BF16 ? 16 : 8))
            return ECF8_ERR_ARG;
        const TabGeo g = table_geometry(t.meta.len);
        if (g.entries > (uint32_t)kTabMax) return ECF8_ERR_UNSUPPORTED;   // never for valid lengths
        DescV& d = dv[i];
        std::memset(&d, 0, sizeof(d));
        d.stream = t.stream;
        d.raw = t.raw;
        d.gaps = t.gaps;
        d.blk_off = t.blk_off;
        d.out = out_base + t.out_offset;
        d.n = t.meta.n;
        d.first_block = blocks;
        if (t.meta.n) blocks += t.meta.n_blocks;
        d.end_block = blocks;
        d.total_bits = t.meta.total_bits;
        d.cdelta = g.cdelta;
        d.p_long = g.p_long;
        d.long_units = g.long_units;
        d.entries = g.entries;
        std::memcpy(d.len, t.meta.len, sizeof(d.len));
        if (t.meta.n && g.entries > tab_n) tab_n = g.entries;
        if (t.meta.n && g.long_units) short_codes = false;
    }
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (count && hipMemcpy(ws + desc_offset(), dv.data(), sizeof(DescV) * count, hipMemcpyHostToDevice) != hipSuccess)
        return ECF8_ERR_HIP;
    // the decode tables depend on the code lengths only: built once here
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    auto* status = reinterpret_cast<unsigned long long*>(ws);
    hipLaunchKernelGGL(ecf8v_clear_kernel, dim3(1), dim3(64), 0, st, status, 2u);
    if (count)
        hipLaunchKernelGGL(ecf8v_table_kernel, dim3((uint32_t)count, (uint32_t)kTableSlices), dim3(256), 0, st,
                           reinterpret_cast<const DescV*>(ws + desc_offset()),
                           reinterpret_cast<uint32_t*>(ws + table_offset(count)), fmt);
    if (hipGetLastError() != hipSuccess || hipStreamSynchronize(st) != hipSuccess) return ECF8_ERR_HIP;
    plan->workspace = workspace;
    plan->workspace_bytes = workspace_bytes;
    plan->total_blocks = blocks;
    plan->count = (uint32_t)count;
    plan->format = fmt;
    plan->threads_per_block = tb;
    plan->table_entries = tab_n;
    plan->short_codes = short_codes ? 1u : 0u;
    uint32_t slots = 1;
    if (blocks) {
        int rc = kernel_slots(fmt, tb, decode_lds_bytes(tab_n), short_codes, &slots);
        if (rc) return rc;
    }
    plan->grid = (uint32_t)(blocks < slots ? (blocks ? blocks : 1) : slots);
    return ECF8_OK;
}

namespace {

int run_plan(const ecf8v_plan* plan, void* hip_stream, hipEvent_t start, hipEvent_t stop)
{
    if (!plan || !plan->workspace || plan->grid == 0) return ECF8_ERR_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    uint8_t* ws = static_cast<uint8_t*>(plan->workspace);
    auto* status = reinterpret_cast<unsigned long long*>(ws);
    const DescV* descs = reinterpret_cast<const DescV*>(ws + desc_offset());
    uint32_t* tables = reinterpret_cast<uint32_t*>(ws + table_offset((int)plan->count));
    if (plan->count == 0 || plan->total_blocks == 0) return ECF8_OK;
    const uint32_t tb = plan->threads_per_block;
    const void* k = pick_kernel(plan->format, tb, plan->short_codes != 0);
    if (!k) return ECF8_ERR_UNSUPPORTED;
    int count = (int)plan->count;
    uint64_t total = plan->total_blocks;
    uint32_t tab_n = plan->table_entries;
    if (tab_n < (uint32_t)kTabMin || tab_n > (uint32_t)kTabMax || (tab_n & 3)) return ECF8_ERR_ARG;
    void* args[] = {(void*)&descs, (void*)&count, (void*)&tables, (void*)&total, (void*)&status, (void*)&tab_n};
    const hipError_t e = start || stop
                             ? hipExtLaunchKernel(k, dim3(plan->grid), dim3(tb), args, decode_lds_bytes(tab_n), st,
                                                  start, stop, 0)
                             : hipLaunchKernel(k, dim3(plan->grid), dim3(tb), args, decode_lds_bytes(tab_n), st);
    if (e != hipSuccess) return ECF8_ERR_HIP;
    return check(hipGetLastError());
}

}  // namespace

extern "C" int ecf8v_decode_run(const ecf8v_plan* plan, void* hip_stream)
{
    return run_plan(plan, hip_stream, nullptr, nullptr);
}

extern "C" int ecf8v_decode_run_timed(const ecf8v_plan* plan, void* hip_stream, void* start_event, void* stop_event)
{
    return run_plan(plan, hip_stream, reinterpret_cast<hipEvent_t>(start_event),
                    reinterpret_cast<hipEvent_t>(stop_event));
}

extern "C" int ecf8v_decode_status(const void* workspace, void* hip_stream, uint64_t* bad_blocks)
{
    if (!workspace || !bad_blocks) return ECF8_ERR_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (hipStreamSynchronize(st) != hipSuccess) return ECF8_ERR_HIP;
    unsigned long long v[2] = {0, 0};
    if (hipMemcpy(v, workspace, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return ECF8_ERR_HIP;
    *bad_blocks = v[0] + v[1];
    if (*bad_blocks) {   // restart the count
        const unsigned long long zero[2] = {0, 0};
        if (hipMemcpy(const_cast<void*>(workspace), zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
            return ECF8_ERR_HIP;
    }
    return *bad_blocks ? ECF8_ERR_CORRUPT : ECF8_OK;
}
