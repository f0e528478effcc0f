// ecf8_decode.hip -- GPU decode of ECF8 streams on MI355X (gfx950, wave64).
//
// Method (ECF8 technical blog, codearts.csdn.net):
//   §3.1.2  table-driven decode of the Huffman-coded exponent;
//   §3.2.1  each thread owns a chunk of the bitstream and a stored gap (the
//           offset of its first codeword), counts its symbols, a block-wide
//           step turns counts into output positions, threads decode
//           cooperatively into shared memory (LDS here) and the block writes
//           its results back;
//   §3.2.2 / §3.3  one reused output buffer, batched decode of resident weights.
// Format: include/ecf8.h.
//
// MI355X-specific design (differs from the pages' CUDA sketch, which targets
// 32-lane warps, 128-thread blocks and an L1-resident two-level 8-bit table):
//   * decode table: one LDS table of packed 4-byte entries indexed by the
//     next 11 stream bits.  Each entry decodes greedily the whole codewords
//     inside the window (up to 4 symbols), ~3.7 symbols per lookup for the
//     weight distributions of interest.  Codes longer than 11 bits (rare) live
//     in a second region indexed by the next 16 bits; one branch-free
//     max(prefix11, prefix16 - c) picks the region (canonical codes put every
//     long code at the top of the code space).  The table is built per tensor
//     on the GPU from the 16 code lengths by a small kernel and copied to LDS
//     by each persistent workgroup when its tensor changes.
//   * chunks: 16 bytes per lane, 256 lanes (4 wave64s) per block; the lane's
//     chunk plus one look-ahead dword are byte-swapped into LDS in word-major
//     order (word k of every lane is one contiguous row), so the window reads
//     of a wave hit 64 distinct banks whatever bit position each lane is at;
//     a 32-bit window is one ds_read2st64 + one v_alignbit.
//   * one walk: the count pass records each lookup's table entry in registers
//     (four lookups per wave-uniform step, so the record index is static) and
//     the decode pass replays them; only lanes with more lookups walk again.
//   * counts -> positions: wave64 inclusive scan with DPP row shifts and
//     readlane row carries, then a 4-entry cross-wave LDS prefix.
//   * decode: the recorded entries are OR-ed two at a time as packed nibbles
//     into the cleared LDS staging area at the scanned nibble positions.  A
//     lane's last lookup may decode a few codewords that belong to the next
//     lane; they are the same symbols at the same positions, so OR-ing them
//     twice is exact.  The stream rows share memory with the staging.
//   * write back: 16 elements per lane-step: 8 bytes of exponent nibbles from
//     LDS, 8 bytes of the sign/mantissa plane from HBM (non-temporal loads
//     issued when the block starts, in flight during the count, scan and
//     decode), SWAR byte assembly, one non-temporal 16-byte store; byte stores
//     only at the two ragged block edges.  The next block's inputs are taken
//     into registers before the stores are issued.
//   * streaming loads and stores are buffer instructions (SGPR descriptors,
//     32-bit offsets, hardware range checks); one persistent dispatch walks
//     all blocks of all tensors of a batch at 6 workgroups per CU;
//   * wave priority rises through a block (count 1, scan and decode 2,
//     write-back 3), so the wave of a SIMD nearest its stores issues first.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "ecf8.h"

namespace {

constexpr int kWin = 11;                                            // primary window bits
constexpr int kLongPrefixMax = 8;                                   // prefixes of codes > kWin bits
constexpr int kTableMax = (1 << kWin) + ((1 << (16 - kWin)) - 1) * kLongPrefixMax;  // 2296
constexpr uint32_t kTabStride = 2304;                               // entries per table array
constexpr int kChunk = 16;                                          // C
constexpr int kLanes = 256;                                         // TB
constexpr uint64_t kStatusBytes = 256;
constexpr int kTableThreads = 256;
constexpr int kNibPrefetch = 4;                                     // write-back groups prefetched per lane

// Device descriptor of one tensor (workspace resident).
struct alignas(16) DevDesc {
    const uint8_t* stream;
    const uint8_t* nibbles;
    const uint8_t* gaps;
    const uint64_t* blk_off;
    uint8_t* out;
    uint64_t n;
    uint64_t total_bits;
    uint64_t block_begin;     // first global block of this tensor in the batch
    uint64_t block_end;       // one past its last global block
    uint8_t len[16];
    // derived on the GPU by the table kernel
    uint64_t lenpack;         // 4 bits per symbol: code length - 1
    uint32_t p_long;          // first 11-bit prefix of a code longer than 11 bits
    int32_t cdelta;           // 31 * p_long (second-region offset)
    uint32_t entries;         // table entries in use
    uint32_t pad0;
    uint64_t pad1[2];
};
static_assert(sizeof(DevDesc) == 128, "descriptor layout");

uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

uint64_t desc_offset() { return kStatusBytes; }
uint64_t table_offset(int count) { return kStatusBytes + round_up((uint64_t)count * sizeof(DevDesc), 256); }
constexpr uint64_t kTableBytes = kTabStride * sizeof(uint32_t);        // one packed dword per entry
constexpr int kMaxSymPerEntry = 4;                                  // symbols decoded per lookup, at most

// Global-memory accessors: descriptor pointers are generic; casting them to
// the global address space makes the compiler emit global_* (not flat_*)
// instructions, which only touch the vector-memory counter.
#define ECF8_GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <class T>
__device__ __forceinline__ T gld(const T* p) { return *(const ECF8_GLOBAL T*)(p); }
__device__ __forceinline__ uint4 gld4(const void* p)
{
    const u32x4 v = *(const ECF8_GLOBAL u32x4*)(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Buffer resources for the streaming loads and stores of the decode kernel: a
// wave-uniform base and byte size in SGPRs, 32-bit per-lane byte offsets, and
// the hardware range check (a load past the end reads 0, a store past the end
// is dropped).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;   // raw, untyped dword access (gfx9 descriptor word 3)
// The decoded output is written once and not read back by this kernel: its
// 16-byte stores carry the non-temporal hint (cache-policy bit 1), which
// measured faster than the default, and so do the sign/mantissa plane loads
// (read once); the stream loads keep the default policy (their neighbouring
// lines are reused from L2 by the look-ahead reads).
constexpr int kNonTemporal = 2;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint64_t bytes)
{
    const uint32_t nr = bytes < 0xFFFFFFFFull ? (uint32_t)bytes : 0xFFFFFFFFu;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nr, kRsrcWord3);
}
__device__ __forceinline__ uint32_t bld1(Rsrc r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bld(Rsrc r, uint32_t off, uint32_t soff = 0)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
}
__device__ __forceinline__ uint2 bld2(Rsrc r, uint32_t off, uint32_t soff = 0)
{
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 bld4(Rsrc r, uint32_t off)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void bst4(Rsrc r, uint32_t off, uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    u32x4 v;
    v.x = a; v.y = b; v.z = c; v.w = d;
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kNonTemporal);
}
__device__ __forceinline__ void bst1(Rsrc r, uint32_t off, uint8_t v)
{
    __builtin_amdgcn_raw_buffer_store_b8(v, r, off, 0, 0);
}

// ------------------------------------------------------------ table kernel
// Grid (tensors, kTableSlices): workgroup (i, j) builds entries
// [256 j, 256 j + 256) of tensor i's table, one entry per lane.  Canonical
// codes occupy consecutive ranges of the left-justified 16-bit code space in
// (length, symbol) order, so symbol s starts at the sum of 2^(16 - len) over
// the symbols before it; each of 16 lanes computes one symbol's range.
// Entry layout (one dword, so a lookup is a single 4-byte LDS read):
//   bits  7..0   bits consumed (1..16)
//   bits 15..8   4 * symbols decoded (0..16)
//   bits 31..16  the symbols as nibbles, first symbol in bits 19..16.
constexpr int kTableSlices = (kTableMax + kTableThreads - 1) / kTableThreads;   // 9

__global__ __launch_bounds__(kTableThreads) void ecf8_table_kernel(DevDesc* __restrict__ descs,
                                                                   uint32_t* __restrict__ tables)
{
    __shared__ uint32_t s_start[16];   // canonical order: left-justified start of the k-th codeword range
    __shared__ uint32_t s_len[16];
    __shared__ uint32_t s_sym[16];
    __shared__ uint32_t s_k;
    DevDesc* d = descs + blockIdx.x;
    const int tid = threadIdx.x;
    if (tid < 16) {
        const uint32_t l = d->len[tid];
        uint32_t rank = 0, start = 0, k = 0, plong_units = 0;
        for (int u = 0; u < 16; ++u) {
            const uint32_t lu = d->len[u];
            if (!lu) continue;
            k++;
            if (lu <= (uint32_t)kWin) plong_units += 1u << (16 - lu);
            if (l && (lu < l || (lu == l && u < tid))) {
                rank++;
                start += 1u << (16 - lu);
            }
        }
        if (l) {
            s_start[rank] = start;
            s_len[rank] = l;
            s_sym[rank] = tid;
        }
        if (tid == 0) {
            s_k = k;
            // every code of at most kWin bits precedes the long ones, so the
            // first long prefix is the total space of the short codes
            const uint32_t p_long = plong_units >> (16 - kWin);
            uint32_t cdelta = ((1u << (16 - kWin)) - 1) * p_long;
            uint32_t entries = 65536u - cdelta;      // <= kTableMax for every complete code
            if (entries > (uint32_t)kTableMax) entries = kTableMax;
            if (blockIdx.y == 0) {
                uint64_t lenpack = 0;
                for (int u = 0; u < 16; ++u)
                    if (d->len[u]) lenpack |= (uint64_t)((d->len[u] - 1) & 15) << (4 * u);
                d->lenpack = lenpack;
                d->p_long = p_long;
                d->cdelta = (int32_t)cdelta;
                d->entries = entries;
            }
        }
    }
    __syncthreads();
    const int k = (int)s_k;
    uint32_t plong_units = 0;
    for (int u = 0; u < 16; ++u) {
        const uint32_t lu = d->len[u];
        if (lu && lu <= (uint32_t)kWin) plong_units += 1u << (16 - lu);
    }
    const uint32_t p_long = plong_units >> (16 - kWin);
    const uint32_t cdelta = ((1u << (16 - kWin)) - 1) * p_long;
    uint32_t entries = 65536u - cdelta;
    if (entries > (uint32_t)kTableMax) entries = kTableMax;
    const uint32_t idx = blockIdx.y * kTableThreads + tid;
    if (idx >= entries) return;
    uint32_t v, known;
    if (idx < p_long) {
        v = idx << (16 - kWin);
        known = kWin;
    } else {
        v = idx + cdelta;
        known = 16;
    }
    uint32_t pos = 0, ns = 0, sy = 0;
    while (k > 0 && ns < (uint32_t)kMaxSymPerEntry && pos < known) {
        const uint32_t x = (v << pos) & 0xFFFFu;
        int lo = 0, hi = k;
        while (hi - lo > 1) {
            int mid = (lo + hi) >> 1;
            if (s_start[mid] <= x) lo = mid;
            else hi = mid;
        }
        const uint32_t l = s_len[lo];
        if (x >= s_start[lo] + (1u << (16 - l))) break;   // outside an incomplete code
        if (pos + l > known) break;                          // codeword not fully visible
        sy |= s_sym[lo] << (4 * ns);
        ns++;
        pos += l;
    }
    tables[(uint64_t)blockIdx.x * kTabStride + idx] = (pos ? pos : 1u) | ((4 * ns) << 8) | (sy << 16);
}

// ------------------------------------------------------------ helpers
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane)
{
    // Hillis-Steele inside each 16-lane DPP row, then carry row totals with readlane.
    v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 15);
    const uint32_t r1 = __builtin_amdgcn_readlane(v, 31);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane >> 4;
    v += (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
    return v;
}

// (a & mask) | (b & ~mask) as one v_bfi_b32 (the compiler otherwise splits it
// into and/or sequences)
__device__ __forceinline__ uint32_t bitsel(uint32_t mask, uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(mask), "v"(a), "v"(b));
    return r;
}

// 8 exponent nibbles (e) + 8 sign/mantissa nibbles (nm), element i in nibble i,
// -> 8 FP8 bytes: byte = (s << 7) | (e << 3) | m with nm = (s << 3) | m.
__device__ __forceinline__ uint2 assemble8(uint32_t e, uint32_t nm)
{
    const uint32_t nev = bitsel(0xF0F0F0F0u, nm << 4, nm);   // byte j: nibble 2j in both halves
    const uint32_t nod = bitsel(0x0F0F0F0Fu, nm >> 4, nm);   // byte j: nibble 2j+1 in both halves
    const uint32_t ev = bitsel(0x78787878u, e << 3, nev);    // elements 0,2,4,6
    const uint32_t od = bitsel(0x78787878u, e >> 1, nod);    // elements 1,3,5,7
    uint2 r;
    r.x = __builtin_amdgcn_perm(od, ev, 0x05010400u);         // e0 e1 e2 e3
    r.y = __builtin_amdgcn_perm(od, ev, 0x07030602u);         // e4 e5 e6 e7
    return r;
}

// Write back group g (elements 16g .. 16g+15 of the block-relative range):
// exponent nibbles from the LDS staging, sign/mantissa nibbles nm from HBM.
__device__ __forceinline__ void group_bytes(const uint32_t* s_out, uint32_t g, uint2 nm, uint32_t w[4])
{
    const uint2 ex = reinterpret_cast<const uint2*>(s_out)[g];
    const uint2 r0 = assemble8(ex.x, nm.x);
    const uint2 r1 = assemble8(ex.y, nm.y);
    w[0] = r0.x;
    w[1] = r0.y;
    w[2] = r1.x;
    w[3] = r1.y;
}

// A group fully inside the block's range: one 16-byte store.
__device__ __forceinline__ void write_full(const uint32_t* s_out, Rsrc out_blk, uint32_t g, uint2 nm)
{
    uint32_t w[4];
    group_bytes(s_out, g, nm, w);
    bst4(out_blk, 16u * g, w[0], w[1], w[2], w[3]);
}

// One of the (at most two) ragged edge groups of a block: store only the
// bytes inside [a0, endo).
__device__ __forceinline__ void write_edge(const uint32_t* s_out, Rsrc out_blk, uint32_t g, uint2 nm,
                                           uint32_t a0, uint32_t endo)
{
    uint32_t w[4];
    group_bytes(s_out, g, nm, w);
    const uint32_t e0 = 16u * g;
    const uint32_t kb = e0 < a0 ? a0 - e0 : 0u;
    const uint32_t ke = endo - e0 < 16u ? endo - e0 : 16u;
#pragma unroll
    for (uint32_t q = 0; q < 16; ++q)
        if (q >= kb && q < ke) bst1(out_blk, e0 + q, (uint8_t)(w[q >> 2] >> (8 * (q & 3))));
}

// One table lookup at stream position r (r = 192 - bit position within the
// lane's chunk): 32-bit window from the lane's two LDS rows, then the index
// max(prefix11, prefix16 - cd) into the packed table.
__device__ __forceinline__ uint32_t lookup(const char* s_stream_b, const uint32_t* s_tx, uint32_t col_addr,
                                           uint32_t r, int cd)
{
    // a = col_addr + 4 * kLanes * ((r >> 5) - 2), as one v_and + one v_lshl_add
    static_assert(4 * kLanes == 32 << 5, "row pitch");
    uint32_t a;
    asm("v_lshl_add_u32 %0, %1, 5, %2" : "=v"(a) : "v"(r & 0xE0u), "v"(col_addr - 2u * 4u * kLanes));
    const uint32_t w1 = *reinterpret_cast<const uint32_t*>(s_stream_b + a);
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(s_stream_b + a + 4u * kLanes);
    const uint32_t win = __builtin_amdgcn_alignbit(w0, w1, r);
    const int idx = max((int)(win >> (32 - kWin)), (int)(win >> 16) - cd);
    return s_tx[idx];
}

// OR the symbols of one table entry, as packed nibbles, into the zeroed
// staging at bit offset ob (two dwords: the entry's 16 symbol bits may
// straddle a dword boundary).
__device__ __forceinline__ void emit_symbols(uint32_t* s_out, uint32_t ob, uint32_t ex)
{
    const uint64_t v = (uint64_t)(ex >> 16) << (ob & 31);
    const uint32_t wa = ob >> 5;
    atomicOr(&s_out[wa], (uint32_t)v);
    atomicOr(&s_out[wa + 1], (uint32_t)(v >> 32));
}

// OR the symbols of two consecutive table entries of a lane (an entry of 0
// contributes nothing) into the staging at bit offset ob: their packets joined
// into one bit string of at most 32 bits, spread over two dwords.  Returns the
// bit offset after them.
__device__ __forceinline__ uint32_t emit_pair(uint32_t* s_out, uint32_t ob, uint32_t e0, uint32_t e1)
{
    // p01 = ((e1 >> 16) << n0) | (e0 >> 16), n0 = 4 * symbols of e0 (<= 16, the low
    // five bits of e0 >> 8), with word selects instead of shifts
    const uint32_t n0s = e0 >> 8;
    uint32_t p01;
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1\n\t"
        "v_or_b32_sdwa %0, %0, %3 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
        : "=&v"(p01) : "v"(n0s), "v"(e1), "v"(e0));
    const uint64_t v = (uint64_t)p01 << (ob & 31u);
    const uint32_t wa = ob >> 5;
    atomicOr(&s_out[wa], (uint32_t)v);
    atomicOr(&s_out[wa + 1], (uint32_t)(v >> 32));
    // ob + (4 * symbols of e0) + (4 * symbols of e1), with byte selects
    uint32_t nob;
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD\n\t"
        "v_add_u32_sdwa %0, %3, %0 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
        : "=&v"(nob) : "v"(e0), "v"(ob), "v"(e1));
    return nob;
}

// ------------------------------------------------------------ decode kernel
#ifndef ECF8_RECORDS
#define ECF8_RECORDS 20
#endif
constexpr int kRecords = ECF8_RECORDS;   // table entries recorded per lane by the count pass
static_assert(kRecords % 4 == 0, "records are taken four at a time");

template <int C, int TB>
struct DecodeLds {
    static constexpr int kSlot = C / 4 + 1;                                   // dwords per lane: chunk + look-ahead
    static constexpr int kStreamDw = TB * (kSlot + 1);                        // rows, + one row only read at shift 0
    static constexpr int kOutDw = ((8 * C * TB + 15 + 8 + 16) / 8 + 2 + 3) / 4 * 4;   // nibble staging
    static constexpr int kUnionDw = kOutDw > kStreamDw ? kOutDw : kStreamDw;
    static_assert(kUnionDw % 4 == 0, "cleared as 16-byte words");
};

// Window at bit position p (p < 128 + 16) of a lane's chunk held in registers
// (w[0..3] the chunk as big-endian words, w[4] the look-ahead word).
__device__ __forceinline__ uint32_t reg_window(const uint32_t (&w)[5], uint32_t p)
{
    const uint32_t k = p >> 5;
    uint32_t hi = w[0], lo = w[1];
    if (k == 1) { hi = w[1]; lo = w[2]; }
    if (k == 2) { hi = w[2]; lo = w[3]; }
    if (k >= 3) { hi = w[3]; lo = w[4]; }
    return (uint32_t)(((((uint64_t)hi << 32) | lo) << (p & 31)) >> 32);
}

// Per-block inputs loaded one block ahead (software pipelining of the
// persistent loop: HBM latency overlaps the previous block's decode).  The
// block offsets are loaded lane-parallel (lane 0: blk_off[b], lane 1:
// blk_off[b+1]) and broadcast with readlane where they are first needed, so
// that no wait for the prefetch is forced right after it is issued.
struct BlockIn {
    uint4 sv;          // the lane's 16 stream bytes
    uint32_t la;       // first dword of the next lane's chunk (look-ahead)
    uint32_t gb;       // byte holding the lane's gap
    uint64_t off;      // lane 0: blk_off[b]; lane 1: blk_off[b + 1]
};

// Descriptor fields the prefetch needs, cached in registers per tensor.
struct NextTensor {
    int t;
    uint64_t begin, end, n;
    const uint8_t* stream;
    const uint8_t* gaps;
    const uint64_t* blk_off;
};

__device__ __forceinline__ void fetch_next_tensor(const DevDesc* descs, int t, NextTensor& nt)
{
    const DevDesc* d = descs + t;
    nt.t = t;
    nt.begin = d->block_begin;
    nt.end = d->block_end;
    nt.n = d->n;
    nt.stream = d->stream;
    nt.gaps = d->gaps;
    nt.blk_off = d->blk_off;
}

// Output range of a block: elements [lo, lo + nw), written as 16-element
// groups from the aligned base (a0 = lo - base), `groups` groups in all.
struct BlockGeo {
    uint64_t lo, base, want;
    uint32_t nw, a0, groups;
};

__device__ __forceinline__ BlockGeo block_geo(uint64_t lo_raw, uint64_t hi_raw, uint64_t n, uint32_t cap)
{
    BlockGeo g;
    const uint64_t hi = hi_raw < n ? hi_raw : n;
    g.lo = lo_raw < hi ? lo_raw : hi;
    g.want = hi - g.lo;
    g.nw = g.want < cap ? (uint32_t)g.want : cap;
    g.base = g.lo & ~15ull;
    g.a0 = (uint32_t)(g.lo - g.base);
    g.groups = (g.a0 + g.nw + 15) >> 4;
    return g;
}

// The sign/mantissa plane of a block's groups (8 bytes per 16-element group):
// the range ends with the block, so that loads for groups past it read 0
// without touching memory.
__device__ __forceinline__ Rsrc nibble_rsrc(const uint8_t* nibbles, const BlockGeo& g)
{
    return make_rsrc(nibbles + (g.base >> 1), 8ull * g.groups);
}

// Issue the sign/mantissa plane loads of a block's groups (one 8-byte
// non-temporal load per group, lane tid takes groups tid + k*TB).  The loads
// are issued unconditionally (past the block they read 0) so that the
// compiler can count outstanding memory operations exactly.
template <int TB>
__device__ __forceinline__ void load_nibbles(Rsrc rn, int tid, uint2 (&nv)[kNibPrefetch])
{
#pragma unroll
    for (int k = 0; k < kNibPrefetch; ++k) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rn, 8u * tid, 8u * k * TB, kNonTemporal);
        nv[k] = make_uint2(v.x, v.y);
    }
}

__device__ __forceinline__ void load_block(const NextTensor& nt, uint64_t gblk, int tid, BlockIn& in)
{
    const uint64_t b = gblk - nt.begin;
    // block offsets first: they are the first of these loads to be needed
    const uint2 o = bld2(make_rsrc(nt.blk_off + b, 16), (tid & 1) * 8u);
    in.off = ((uint64_t)o.y << 32) | o.x;
    // the block's chunks and the look-ahead word of its last lane (the stream
    // has 16 bytes past its last block)
    const Rsrc rs = make_rsrc(nt.stream + b * (kLanes * kChunk), kLanes * kChunk + 16);
    in.sv = bld4(rs, tid * kChunk);
    in.la = bld(rs, tid * kChunk + kChunk);
    in.gb = bld1(make_rsrc(nt.gaps + b * (kLanes / 2), kLanes / 2), tid >> 1);
}

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

#ifndef ECF8_MIN_WAVES
#define ECF8_MIN_WAVES 6
#endif

template <int C, int TB>
__global__ __launch_bounds__(TB) __attribute__((amdgpu_waves_per_eu(ECF8_MIN_WAVES))) void ecf8_decode_kernel(const DevDesc* __restrict__ descs, int count,
                                                         uint64_t total_blocks,
                                                         const uint32_t* __restrict__ tables,
                                                         unsigned long long* __restrict__ status)
{
    static_assert(C == kChunk && TB == kLanes, "one instantiation");
    using L = DecodeLds<C, TB>;
    constexpr int kWaves = TB / 64;
    constexpr int S = L::kSlot;
    // One LDS arena: decode table | nibble staging, whose first S * TB dwords
    // double as the stream rows | wave sums.  The stream rows are read only by
    // the count pass and the staging is written only after the block-wide
    // scan, so the two share memory: a lane clears its own rows once it has
    // counted, the write-back clears what the decode wrote, and a barrier at
    // the top of each block orders the previous block's write-back before the
    // new rows are written.
    constexpr int kUnionOff = (int)kTabStride;
    constexpr int kSumOff = kUnionOff + L::kUnionDw;
    __shared__ __align__(256) uint32_t lds[kSumOff + kWaves];
    uint32_t* const s_tx = lds;
    uint32_t* const s_out = lds + kUnionOff;
    uint32_t* const s_stream = lds + kUnionOff;
    uint32_t* const s_wsum = lds + kSumOff;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // Lane words in word-major, reversed order: word k of the lane's chunk
    // (k = 0..S-1, k = S-1 the look-ahead) lives in row S - k, element tid;
    // row S + 1 (staging memory) is only read with a zero funnel shift, and a
    // finished lane may read row 0 (the last table dwords) for a window it drops.  With
    // r = 192 - bitpos, the window pair (word ceil(bitpos/32)-1, next word) is
    // rows (r >> 5) and (r >> 5) - 1, and the funnel shift is r & 31.
    static_assert(S == 5, "r = 192 - bitpos assumes 4 chunk words + look-ahead");
    uint32_t* const col = s_stream - TB + tid;                 // col[row * TB] = row `row`, rows 1..S+1
    const uint32_t col_addr = (uint32_t)tid * 4u;              // byte address of row 1, this lane
    const char* const s_stream_b = reinterpret_cast<const char*>(s_stream);

    uint64_t blk = blockIdx.x;
    if (blk >= total_blocks) return;
    for (int i = tid; i < L::kUnionDw / 4; i += TB) reinterpret_cast<uint4*>(s_out)[i] = make_uint4(0, 0, 0, 0);

    NextTensor nt;
    fetch_next_tensor(descs, 0, nt);
    while (nt.t + 1 < count && blk >= nt.end) fetch_next_tensor(descs, nt.t + 1, nt);
    BlockIn nx;
    load_block(nt, blk, tid, nx);
    int ptens = nt.t;                  // tensor of the prefetched block
    const uint32_t cap = 8u * C * TB;  // staging capacity in elements
    // wait for the first block's loads here, so that at the loop head only the
    // back edge has loads in flight and the compiler can count them exactly
    asm volatile("" ::"v"(nx.sv.x), "v"(nx.la), "v"(nx.gb), "v"((uint32_t)nx.off));

    // fields of the tensor being decoded
    int cur = -1;
    uint64_t c_begin = 0, c_n = 0, c_T = 0, c_lenpack = 0;
    const uint8_t* c_nib = nullptr;
    const uint8_t* c_stream = nullptr;
    uint8_t* c_out = nullptr;
    int c_cd = 0;
    uint32_t c_ok = 0;

    for (; blk < total_blocks; blk += gridDim.x) {
        const BlockIn in = nx;
        if (ptens != cur) {
            const DevDesc* d = descs + ptens;
            c_begin = d->block_begin;
            c_n = d->n;
            c_T = d->total_bits;
            c_lenpack = d->lenpack;
            c_nib = d->nibbles;
            c_stream = d->stream;
            c_out = d->out;
            c_cd = d->cdelta;
            uint32_t ne = d->entries;
            c_ok = ne != 0;                       // 0: tables were never built for this plan
            ne = ne < (uint32_t)kTableMax ? ne : (uint32_t)kTableMax;
            const uint32_t* tx = tables + (uint64_t)ptens * kTabStride;
            // (every lane left the previous decode pass at its closing barrier,
            // so the old table is no longer read).  16-byte loads, at most 3 per
            // lane: each load waits for every memory operation in flight (the
            // previous block's stores too), so fewer, wider loads cost fewer
            // round trips (3% faster than dword loads).
            const uint32_t n4 = (ne + 3) / 4;
            const Rsrc rt = make_rsrc(tx, 16ull * n4);
            for (uint32_t i = tid; i < n4; i += TB)
                reinterpret_cast<u32x4*>(s_tx)[i] = __builtin_amdgcn_raw_buffer_load_b128(rt, 16u * i, 0, 0);
            cur = ptens;
        }
        // the table is in place and every lane has finished the previous block's
        // write-back, whose staging memory the stream rows reuse
        __syncthreads();
        // stage the chunk (big-endian words, reversed order) into the lane's rows
        col[S * TB] = __builtin_bswap32(in.sv.x);
        col[(S - 1) * TB] = __builtin_bswap32(in.sv.y);
        col[(S - 2) * TB] = __builtin_bswap32(in.sv.z);
        col[(S - 3) * TB] = __builtin_bswap32(in.sv.w);
        col[(S - 4) * TB] = __builtin_bswap32(in.la);
        const uint64_t b = blk - c_begin;
        // stream bits of the tensor from this block's start (uniform), then the
        // lane's own: E = bits of its chunk before the end of the stream
        const uint64_t bbits = b * (8ull * C * TB);
        const uint64_t left = (c_T > bbits && c_ok) ? c_T - bbits : 0ull;
        const uint32_t leftc = left < 8ull * C * TB ? (uint32_t)left : 8u * C * TB;
        const uint32_t lstart = (uint32_t)tid * (8u * C);
        const uint32_t E = leftc > lstart ? min(leftc - lstart, 8u * C) : 0u;
        const uint32_t gap = (in.gb >> ((tid & 1) * 4)) & 15u;

        // block output range and its 16-element groups
        const BlockGeo geo = block_geo(lane_u64(in.off, 0), lane_u64(in.off, 1), c_n, cap);
        const uint64_t base = geo.base;
        const uint32_t a0 = geo.a0, nw = geo.nw, groups = geo.groups;
        const uint64_t want = geo.want;
        const Rsrc nib_blk = nibble_rsrc(c_nib, geo);
        // the block's sign/mantissa plane, in flight during the count, scan and
        // decode.  Issued after the previous block's stores (loaded a block
        // ahead instead, they queued behind those stores and held registers
        // across two counts) and before the next block's inputs.
        uint2 nv[kNibPrefetch];
        load_nibbles<TB>(nib_blk, tid, nv);

        // prefetch the next block of this workgroup (after the last block, the
        // current one is re-read: unconditional loads keep the wait counts exact)
        const uint64_t nb = blk + gridDim.x;
        const uint64_t nbe = nb < total_blocks ? nb : blk;
        while (nt.t + 1 < count && nbe >= nt.end) fetch_next_tensor(descs, nt.t + 1, nt);
        load_block(nt, nbe, tid, nx);
        ptens = nt.t;

        // Wave priorities rise through the block: count 1, scan and decode 2,
        // write-back 3, then 0 until the next count.  Among the waves of a SIMD
        // (each from another workgroup, at another point of its block), the one
        // nearest its stores issues first, so stores leave earlier and the
        // next blocks' loads start sooner (4% faster than one raised count).
        __builtin_amdgcn_s_setprio(1);
        // ---- phase 2: count the codewords that start inside [gap, E)
        // The walk runs in steps of four lookups with one wave-uniform exit test
        // per step; a lane that has passed E keeps looking up at its final
        // position but records 0 (no bits, no symbols).  The recorded entries sit
        // in statically indexed registers and are replayed by phase 4, so the
        // stream is walked once (lanes with more than kRecords lookups finish with
        // a plain walk).
        const int cd = c_cd;
        const uint32_t rend = 192u - E;
        const uint32_t r0 = 192u - gap;
        uint32_t rec[kRecords];
        uint32_t r = r0;
        uint32_t cnt4 = 0, lastex = 0;
        bool act = r > rend;
        int nq = 0;                        // four-lookup steps taken (wave-uniform)
#pragma unroll
        for (int q = 0; q < kRecords / 4; ++q) {
            if (__builtin_amdgcn_ballot_w64(act) == 0) break;
            nq = q + 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t e = lookup(s_stream_b, s_tx, col_addr, r, cd);
                const uint32_t em = act ? e : 0u;
                lastex = act ? e : lastex;
                rec[4 * q + j] = em;
                r -= em & 0xFFu;
                cnt4 += (em >> 8) & 0xFFu;
                act = r > rend;
            }
        }
        const uint32_t r_rec = r;          // where the recorded lookups end
        while (r > rend) {
            const uint32_t e = lookup(s_stream_b, s_tx, col_addr, r, cd);
            lastex = e;
            r -= e & 0xFFu;
            cnt4 += (e >> 8) & 0xFFu;
        }
        __builtin_amdgcn_s_setprio(2);
        // the lane's rows are staging memory from here on: leave them cleared
#pragma unroll
        for (int k = 0; k < S; ++k) col[(S - k) * TB] = 0u;
        uint32_t cnt = cnt4 >> 2;
        if (r != r0) {
            // the last lookup (at r + its bit count) may have decoded codewords
            // that start at or after E: keep those starting before E
            const uint32_t ex = lastex;
            const uint32_t ns = (ex >> 10) & 0x3Fu;
            const uint32_t room = r + (ex & 0xFFu) - rend;
            uint32_t sy = ex >> 16, start = 0, keep = 0;
#pragma unroll
            for (int i = 0; i < kMaxSymPerEntry; ++i) {
                if ((uint32_t)i < ns) {
                    keep += start < room ? 1u : 0u;
                    start += (uint32_t)((c_lenpack >> (4 * (sy & 15))) & 15) + 1;
                    sy >>= 4;
                }
            }
            cnt -= ns - keep;
        }

        // the next block's inputs, issued at the top, are taken now, before
        // this block's stores
        asm volatile("" ::"v"(nx.sv.x), "v"(nx.la), "v"(nx.gb), "v"((uint32_t)nx.off));

        // ---- phase 3: block-wide exclusive scan of the counts
        const uint32_t incl = wave_inclusive_scan(cnt, lane);
        if (lane == 63) s_wsum[wave] = incl;
        __syncthreads();
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t sw = s_wsum[w];
            before += (w < wave) ? sw : 0u;
            total += sw;
        }
        const uint32_t pos = before + incl - cnt;

        // ---- phase 4: cooperative decode into the LDS staging (packed nibbles)
        uint32_t ob = (a0 + pos) * 4;      // bit offset of the lane's first nibble in the staging
#pragma unroll
        for (int q = 0; q < kRecords / 4; ++q) {
            if (q >= nq) break;
            ob = emit_pair(s_out, ob, rec[4 * q], rec[4 * q + 1]);
            ob = emit_pair(s_out, ob, rec[4 * q + 2], rec[4 * q + 3]);
        }
        if (r_rec > rend) {
            // lanes with more than kRecords lookups walk the rest from registers
            // (their rows are staging memory now): reload the chunk (L2-resident)
            const uint8_t* sp = c_stream + (b * TB + tid) * kChunk;
            const uint4 cv = gld4(sp);
            const uint32_t w[5] = {__builtin_bswap32(cv.x), __builtin_bswap32(cv.y), __builtin_bswap32(cv.z),
                                   __builtin_bswap32(cv.w), __builtin_bswap32(gld(reinterpret_cast<const uint32_t*>(sp + kChunk)))};
            r = r_rec;
            while (r > rend) {
                const uint32_t win = reg_window(w, 192u - r);
                const int idx = max((int)(win >> (32 - kWin)), (int)(win >> 16) - cd);
                const uint32_t ex = s_tx[idx];
                emit_symbols(s_out, ob, ex);
                ob += (ex >> 8) & 0xFFu;
                r -= ex & 0xFFu;
            }
        }
        __syncthreads();

        __builtin_amdgcn_s_setprio(3);
        // ---- phase 5: write back [lo, lo + nw) as 16-element groups
        if (tid == 0 && (want != total || !c_ok)) atomicAdd(status, 1ull);
        const Rsrc out_blk = make_rsrc(c_out + base, c_n - base);
        const uint32_t endo = a0 + nw;                 // one past the last valid element, group-relative
        const uint32_t first_full = a0 ? 1u : 0u;
        const uint32_t end_full = endo >> 4;           // groups [first_full, end_full) are whole
        // assemble prefetched groups four at a time, then issue their stores back to
        // back: stores share the vector-memory counter with loads, so no wait falls
        // between them
        static_assert(kNibPrefetch % 2 == 0, "write-back batches of two groups");
#pragma unroll
        for (int k0 = 0; k0 < kNibPrefetch; k0 += 2) {
            if (tid + k0 * TB >= end_full) break;
            uint32_t wb[2][4];
#pragma unroll
            for (int k = 0; k < 2; ++k) group_bytes(s_out, tid + (k0 + k) * TB, nv[k0 + k], wb[k]);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t g = tid + (k0 + k) * TB;
                if (g >= first_full && g < end_full)
                    bst4(out_blk, 16u * g, wb[k][0], wb[k][1], wb[k][2], wb[k][3]);
            }
        }
        for (uint32_t g = tid + kNibPrefetch * TB; g < end_full; g += TB)   // blocks of > 16K elements
            write_full(s_out, out_blk, g, bld2(nib_blk, 8u * g));
        // ragged edges: group 0 when the range starts mid-group, group end_full when it ends mid-group
        if (a0 && tid == 0) write_edge(s_out, out_blk, 0, nv[0], a0, endo);
        if (end_full < groups && !(end_full == 0 && a0) && tid == (int)(end_full % TB)) {
            const uint32_t k = end_full / TB;
            uint2 nm = nv[0];
#pragma unroll
            for (int q = 1; q < kNibPrefetch; ++q)
                if (k == (uint32_t)q) nm = nv[q];
            if (k >= (uint32_t)kNibPrefetch) nm = bld2(nib_blk, 8u * end_full);
            write_edge(s_out, out_blk, end_full, nm, a0, endo);
        }
        __builtin_amdgcn_s_setprio(0);
        // clear the staging the decode wrote: groups [0, zend) cover every
        // nibble OR-ed in, the codewords a last lane decodes past the end included
        // (each group is cleared by the lane that read it above)
        {
            const uint32_t zend0 = (a0 + total + 3u + 15u) >> 4;
            const uint32_t zend = zend0 < (uint32_t)(L::kOutDw / 2) ? zend0 : (uint32_t)(L::kOutDw / 2);
            for (uint32_t g = tid; g < zend; g += TB) reinterpret_cast<uint2*>(s_out)[g] = make_uint2(0u, 0u);
        }
    }
}

// ------------------------------------------------------------ host helpers
struct DeviceInfo {
    int cus = 0;
    int occupancy = 0;
};

std::mutex g_dev_mu;
std::vector<DeviceInfo> g_dev;

int device_info(DeviceInfo* out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ECF8_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
    DeviceInfo& di = g_dev[dev];
    if (di.cus == 0) {
        int cus = 0, occ = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return ECF8_ERR_HIP;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &occ, reinterpret_cast<const void*>(ecf8_decode_kernel<kChunk, kLanes>), kLanes, 0) != hipSuccess)
            return ECF8_ERR_HIP;
        di.cus = cus > 0 ? cus : 1;
        di.occupancy = occ > 0 ? occ : 1;
    }
    *out = di;
    return ECF8_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" uint64_t ecf8_workspace_bytes(int count)
{
    if (count < 0) return 0;
    return table_offset(count) + (uint64_t)count * kTableBytes;
}

extern "C" int ecf8_decode_prepare(const ecf8_tensor_desc* descs, int count, uint8_t* out_base,
                                   void* workspace, uint64_t workspace_bytes, void* hip_stream,
                                   ecf8_plan* plan)
{
    if (!plan || count < 0 || (count > 0 && !descs)) return ECF8_ERR_ARG;
    std::memset(plan, 0, sizeof(*plan));
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < ecf8_workspace_bytes(count))
        return ECF8_ERR_WORKSPACE;
    std::vector<unsigned char> host(table_offset(count) - 0, 0);   // status + descriptors
    DevDesc* hd = reinterpret_cast<DevDesc*>(host.data() + desc_offset());
    uint64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        const ecf8_tensor_desc& td = descs[i];
        const ecf8_meta& m = td.meta;
        int rc = ecf8_validate_meta(&m);
        if (rc) return rc;
        if (m.chunk_bytes != (uint32_t)kChunk || m.threads_per_block != (uint32_t)kLanes)
            return ECF8_ERR_UNSUPPORTED;
        if (m.n > 0) {
            if (!out_base || !td.s.stream || !td.s.nibbles || !td.s.gaps || !td.s.blk_off) return ECF8_ERR_ARG;
            if (!aligned(td.s.stream, 16) || !aligned(td.s.nibbles, 8) || !aligned(td.s.blk_off, 8) ||
                !aligned(out_base + td.out_offset, 16))
                return ECF8_ERR_ARG;
        }
        DevDesc& dd = hd[i];
        dd.stream = td.s.stream;
        dd.nibbles = td.s.nibbles;
        dd.gaps = td.s.gaps;
        dd.blk_off = td.s.blk_off;
        dd.out = out_base ? out_base + td.out_offset : nullptr;
        dd.n = m.n;
        dd.total_bits = m.total_bits;
        dd.block_begin = blocks;
        blocks += m.n_blocks;
        dd.block_end = blocks;
        for (int s = 0; s < 16; ++s) dd.len[s] = m.cb.len[s];
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (hipMemcpyAsync(workspace, host.data(), host.size(), hipMemcpyHostToDevice, st) != hipSuccess)
        return ECF8_ERR_HIP;
    DeviceInfo di;
    int rc = device_info(&di);
    if (rc) return rc;
    uint64_t grid = (uint64_t)di.cus * (uint64_t)di.occupancy;
    if (grid > blocks) grid = blocks;
    plan->workspace = workspace;
    plan->workspace_bytes = workspace_bytes;
    plan->total_blocks = blocks;
    plan->count = (uint32_t)count;
    plan->chunk_bytes = kChunk;
    plan->threads_per_block = kLanes;
    plan->grid = (uint32_t)grid;
    return ECF8_OK;
}

namespace {

int check_plan(const ecf8_plan* plan)
{
    if (!plan) return ECF8_ERR_ARG;
    if (plan->count == 0 || plan->total_blocks == 0) return ECF8_OK;
    if (!plan->workspace || plan->workspace_bytes < ecf8_workspace_bytes((int)plan->count))
        return ECF8_ERR_WORKSPACE;
    if (plan->chunk_bytes != (uint32_t)kChunk || plan->threads_per_block != (uint32_t)kLanes || plan->grid == 0)
        return ECF8_ERR_ARG;
    return ECF8_OK;
}

}  // namespace

extern "C" int ecf8_build_tables(const ecf8_plan* plan, void* hip_stream)
{
    int rc = check_plan(plan);
    if (rc || plan->count == 0 || plan->total_blocks == 0) return rc;
    unsigned char* ws = static_cast<unsigned char*>(plan->workspace);
    DevDesc* dd = reinterpret_cast<DevDesc*>(ws + desc_offset());
    uint32_t* tables = reinterpret_cast<uint32_t*>(ws + table_offset((int)plan->count));
    hipLaunchKernelGGL(ecf8_table_kernel, dim3(plan->count, kTableSlices), dim3(kTableThreads), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), dd, tables);
    return hipGetLastError() == hipSuccess ? ECF8_OK : ECF8_ERR_HIP;
}

extern "C" int ecf8_decode_blocks(const ecf8_plan* plan, void* hip_stream)
{
    int rc = check_plan(plan);
    if (rc || plan->count == 0 || plan->total_blocks == 0) return rc;
    unsigned char* ws = static_cast<unsigned char*>(plan->workspace);
    DevDesc* dd = reinterpret_cast<DevDesc*>(ws + desc_offset());
    uint32_t* tables = reinterpret_cast<uint32_t*>(ws + table_offset((int)plan->count));
    auto* status = reinterpret_cast<unsigned long long*>(ws);
    hipLaunchKernelGGL((ecf8_decode_kernel<kChunk, kLanes>), dim3(plan->grid), dim3(kLanes), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), dd, (int)plan->count, plan->total_blocks,
                       tables, status);
    return hipGetLastError() == hipSuccess ? ECF8_OK : ECF8_ERR_HIP;
}

extern "C" int ecf8_decode_run(const ecf8_plan* plan, void* hip_stream)
{
    int rc = ecf8_build_tables(plan, hip_stream);
    if (rc) return rc;
    return ecf8_decode_blocks(plan, hip_stream);
}

extern "C" int ecf8_decode_batched(const ecf8_tensor_desc* descs, int count, uint8_t* out_base,
                                   void* workspace, uint64_t workspace_bytes, void* hip_stream)
{
    ecf8_plan plan;
    int rc = ecf8_decode_prepare(descs, count, out_base, workspace, workspace_bytes, hip_stream, &plan);
    if (rc) return rc;
    return ecf8_decode_run(&plan, hip_stream);
}

extern "C" int ecf8_decode(const ecf8_stream* s, const ecf8_meta* meta, uint8_t* out_fp8, uint64_t n,
                           void* workspace, uint64_t workspace_bytes, void* hip_stream)
{
    if (!s || !meta) return ECF8_ERR_ARG;
    if (n != meta->n) return ECF8_ERR_SIZE;
    ecf8_tensor_desc td;
    td.s = *s;
    td.meta = *meta;
    td.out_offset = 0;
    return ecf8_decode_batched(&td, 1, out_fp8, workspace, workspace_bytes, hip_stream);
}

extern "C" int ecf8_decode_status(const void* workspace, void* hip_stream, uint64_t* bad_blocks)
{
    if (!workspace || !bad_blocks) return ECF8_ERR_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (hipStreamSynchronize(st) != hipSuccess) return ECF8_ERR_HIP;
    unsigned long long v = 0;
    if (hipMemcpy(&v, workspace, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return ECF8_ERR_HIP;
    *bad_blocks = v;
    return v ? ECF8_ERR_CORRUPT : ECF8_OK;
}
