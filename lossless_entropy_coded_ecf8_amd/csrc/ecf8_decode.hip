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
//     long code at the top of the code space).  Each tensor's table is built
//     from its 16 code lengths once per plan (the codebooks are fixed), in LDS
//     by a small kernel (a first-symbol table of the 11-bit windows, chained)
//     that stores it; each persistent decode workgroup copies it into LDS
//     when its tensor changes, so a decode run is one dispatch.
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
//     all blocks of all tensors of a batch at 6 workgroups per CU, each
//     workgroup every G-th block, or, over dispatches long enough for the
//     workgroups to drift apart, in claims of consecutive blocks taken from a
//     counter (the claimed order, chosen per plan);
//   * wave priority rises through a block (count 1, scan and decode 2,
//     write-back 3), so the wave of a SIMD nearest its stores issues first.
#include <hip/hip_ext.h>
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
constexpr int kChunk = 16;                                          // the tuned shape: C
constexpr int kLanes = 256;                                         // and TB
constexpr uint64_t kStatusBytes = 256;
// Inside the status area: the block-check counter at 0, the two counters of
// the claimed block order at kSchedOffset (zeroed when a plan is prepared;
// each run leaves them zero).
constexpr uint64_t kSchedOffset = 64;
// The claimed order: blocks per claim, and the blocks per workgroup from which
// a plan takes it (measured on MoE layers of 32 to 256 experts, 66 to 515
// blocks per workgroup: 3-10% faster than the static order in claims of 4;
// claims of 2 queue on the counter; the Llama-3-70B block, 38 blocks per
// workgroup, is 4% slower in claims).
constexpr uint32_t kClaimBlocks = 4;
constexpr uint32_t kClaimBlocksMax = 1024;
constexpr uint64_t kClaimMinBlocksPerWg = 64;
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
    // derived from len[] on the host when the plan is prepared
    uint64_t lenpack;         // 4 bits per symbol: code length - 1
    uint32_t p_long;          // first 11-bit prefix of a code longer than 11 bits
    int32_t cdelta;           // 31 * p_long (second-region offset)
    uint32_t entries;         // table entries in use
    uint16_t start[16];       // canonical code of each symbol, left-justified to 16 bits
    uint32_t pad;
};
static_assert(sizeof(DevDesc) == 144, "descriptor layout");

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

// ------------------------------------------------------------ helpers
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v)
{
    // Hillis-Steele inside each 16-lane DPP row, then the row totals carried
    // with the row broadcasts: lane 15 of rows 0 and 2 into rows 1 and 3,
    // then lane 31 into rows 2 and 3 (rows a broadcast does not write add 0).
    v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1 and 3
    v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2 and 3
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
// The staging group is cleared once read (the next block ORs into it); each
// group is read, and so cleared, by one lane.
__device__ __forceinline__ void group_bytes(uint32_t* s_out, uint32_t g, uint2 nm, uint32_t w[4])
{
    const uint2 ex = reinterpret_cast<const uint2*>(s_out)[g];
    // two dword stores of one zero register (a 64-bit store would hold a
    // zero register pair live through the write-back)
    s_out[2 * g] = 0u;
    s_out[2 * g + 1] = 0u;
    const uint2 r0 = assemble8(ex.x, nm.x);
    const uint2 r1 = assemble8(ex.y, nm.y);
    w[0] = r0.x;
    w[1] = r0.y;
    w[2] = r1.x;
    w[3] = r1.y;
}

// A group fully inside the block's range: one 16-byte store.
__device__ __forceinline__ void write_full(uint32_t* s_out, Rsrc out_blk, uint32_t g, uint2 nm)
{
    uint32_t w[4];
    group_bytes(s_out, g, nm, w);
    bst4(out_blk, 16u * g, w[0], w[1], w[2], w[3]);
}

// One of the (at most two) ragged edge groups of a block: store only the
// bytes inside [a0, endo).
__device__ __forceinline__ void write_edge(uint32_t* s_out, Rsrc out_blk, uint32_t g, uint2 nm,
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

// Table index of a 32-bit window: max(prefix11, prefix16 - cd), clamped to
// the last entry.  For every complete code the unclamped index is already
// below the built entry count; the clamp matters for the one incomplete code
// that validates (a single symbol of length 1), whose windows starting with a
// 1 bit are no codeword: there it selects an entry that consumes one bit and
// decodes nothing (every built entry consumes at least one bit), so a
// corrupted single-symbol stream still ends each walk and is counted by the
// block check.  prefix11 <= 2047 < kTableMax - 1, so the clamp is one
// v_med3_i32 in place of the v_max_i32.  kShort: the code has no codeword
// longer than kWin bits (see kShortCd), and the index is prefix11.
template <bool kShort = false>
__device__ __forceinline__ int table_index(uint32_t win, int cd)
{
    const int a = (int)(win >> (32 - kWin));
    if constexpr (kShort) return a;
    const int b = (int)(win >> 16) - cd;
    int m;
    asm("v_med3_i32 %0, %1, %2, %3" : "=v"(m) : "v"(a), "v"(b), "v"(kTableMax - 1));
    return m;
}

// cdelta of a complete code with no codeword longer than kWin bits (every
// 11-bit prefix short): its second region is empty and max(prefix11,
// prefix16 - cd) is prefix11, so table_index<true> (one shift) gives the
// same entry as the general form.
constexpr int kShortCd = ((1 << (16 - kWin)) - 1) << kWin;

// log2 of TB / 8: (r & ~31) << kPitchShift<TB> = (r >> 5) * (4 * TB), the byte
// offset of row r >> 5 in rows of TB dwords
template <int TB>
constexpr int kPitchShift = TB == 64 ? 3 : TB == 128 ? 4 : TB == 256 ? 5 : TB == 512 ? 6 : 7;

// The 32-bit window at stream position r (r = 32 (S + 1) - bit position
// within the lane's chunk, S = C / 4 + 1 words per lane), from the lane's two
// LDS rows.
template <int TB>
__device__ __forceinline__ uint32_t window(const char* s_stream_b, uint32_t col_addr, uint32_t r)
{
    // a = col_addr + 4 * TB * ((r >> 5) - 2), as one v_and + one v_lshl_add
    static_assert((4 * TB) == (32 << kPitchShift<TB>), "row pitch");
    uint32_t a;
    asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(a) : "v"(r & ~31u), "i"(kPitchShift<TB>), "v"(col_addr - 2u * 4u * TB));
    const uint32_t w1 = *reinterpret_cast<const uint32_t*>(s_stream_b + a);
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(s_stream_b + a + 4u * TB);
    return __builtin_amdgcn_alignbit(w0, w1, r);
}

// One table lookup at stream position r: the window, then the index
// max(prefix11, prefix16 - cd) into the packed table.
template <int TB>
__device__ __forceinline__ uint32_t lookup(const char* s_stream_b, const uint32_t* s_tx, uint32_t col_addr,
                                           uint32_t r, int cd)
{
    return s_tx[table_index(window<TB>(s_stream_b, col_addr, r), cd)];
}

// The window after entry e: win << (bits e consumes), as one shift with a
// byte select.  An entry consumes at most 16 bits, so the shifted window
// still holds the 16 stream bits a lookup reads (the bits shifted in are
// zeros, past what the index looks at).
__device__ __forceinline__ uint32_t window_after(uint32_t win, uint32_t e)
{
    uint32_t w;
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
        : "=v"(w) : "v"(e), "v"(win));
    return w;
}

// acc + (e & 0xFF) as one byte-select add
__device__ __forceinline__ uint32_t add_byte0(uint32_t acc, uint32_t e)
{
    uint32_t r;
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:DWORD"
        : "=v"(r) : "v"(e), "v"(acc));
    return r;
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

// OR the symbols of two consecutive records of a lane (the entries of a pair
// of lookups; the second's byte 0 holds the pair's nibble count, and records
// of a lane past its end are 0) into the staging at bit offset ob: their packets joined
// into one bit string of at most 32 bits, which covers dword ob / 32 and, when
// it crosses, part of the next.  Only the first of those dwords is written
// here, together with `carry`, the spill of the previous pair into this same
// dword; this pair's own spill is returned in `carry` for the next pair (or
// the final flush).  A pair adds at most 32 bits, so the next pair starts in
// this dword or the next one, and a spill is non-zero only if it starts in the
// next: the carry always lands in the dword it belongs to, with one LDS atomic
// per pair instead of two.  Returns the bit offset after the pair.
__device__ __forceinline__ uint32_t emit_pair(uint32_t* s_out, uint32_t ob, uint32_t e0, uint32_t e1,
                                              uint32_t& carry)
{
    // p01 = ((e1 >> 16) << n0) | (e0 >> 16), n0 = 4 * symbols of e0 (<= 16: the
    // shift takes the low five bits of e0 itself), with word selects
    const uint32_t n0s = e0;
    uint32_t p01;
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1\n\t"
        "v_or_b32_sdwa %0, %0, %3 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
        : "=&v"(p01) : "v"(n0s), "v"(e1), "v"(e0));
    const uint64_t v = (uint64_t)p01 << (ob & 31u);
    atomicOr(&s_out[ob >> 5], (uint32_t)v | carry);
    carry = (uint32_t)(v >> 32);
    // ob + 4 * symbols of the pair: byte 0 of the second record holds it
    return add_byte0(ob, e1);
}

// ------------------------------------------------------------ decode kernel
#ifndef ECF8_RECORDS
#define ECF8_RECORDS 20
#endif
constexpr int kRecords = ECF8_RECORDS;   // table entries recorded per lane by the count pass
#ifndef ECF8_STEP
#define ECF8_STEP 4
#endif
constexpr int kStep = ECF8_STEP;         // lookups per wave-uniform step of the count pass
static_assert(kRecords % kStep == 0 && kStep % 2 == 0, "records are taken a step at a time, emitted in pairs");

// The count pass in wave-uniform steps of kStep lookups, unrolled at compile
// time so that every record index is static (the records stay in registers):
// steps Q .. QEND - 1.  Masked steps: a lane past its end keeps looking up at
// its final position but records 0 (no bits, no symbols), and the walk ends
// when no lane of the wave is active.  Unmasked steps are for lookups every
// lane is sure to take (see kSureSteps).
template <int TB, int Q, int QEND, bool kMasked, bool kShort>
__device__ __forceinline__ void count_steps(const char* s_stream_b, const uint32_t* s_tx, uint32_t col_addr, int cd,
                                            uint32_t rend, uint32_t& r, uint32_t& cnt4, uint32_t& lastex, bool& act,
                                            int& nq, uint32_t (&rec)[kRecords])
{
    if constexpr (Q < QEND) {
        if constexpr (kMasked) {
            if (__builtin_amdgcn_ballot_w64(act) == 0) return;
        }
        nq = Q + 1;
        uint32_t win = 0;
        // lookups in pairs: the second takes its window from the first's,
        // shifted by the bits the first consumed (no LDS read of the rows)
#pragma unroll
        for (int j = 0; j < kStep; ++j) {
            if (j % 2 == 0) win = window<TB>(s_stream_b, col_addr, r);
            else win = window_after(win, rec[kStep * Q + j - 1]);
            const uint32_t e = s_tx[table_index<kShort>(win, cd)];
            uint32_t em = e;
            if constexpr (kMasked) {
                em = act ? e : 0u;
                lastex = act ? e : lastex;
            }
            r -= (em >> 8) & 0xFFu;
            if (j % 2 == 0) {
                rec[kStep * Q + j] = em;
            } else {
                // the pair's second record carries the pair's nibble count in
                // its byte 0 (4 * symbols of both, at most 32: no carry into
                // the bit count), which the decode pass adds in one step
                rec[kStep * Q + j] = add_byte0(em, rec[kStep * Q + j - 1]);
                cnt4 = add_byte0(cnt4, rec[kStep * Q + j]);
            }
            if constexpr (kMasked) act = r > rend;
        }
        count_steps<TB, Q + 1, QEND, kMasked, kShort>(s_stream_b, s_tx, col_addr, cd, rend, r, cnt4, lastex, act, nq,
                                                      rec);
    }
}

// Steps every lane takes when its chunk is whole (E = 8C): the walk starts at
// most 15 bits in and a lookup consumes at most 16 bits, so lookup k starts at
// most at bit 15 + 16k, before 8C for every k < C / 2.
template <int C>
constexpr int kSureSteps = (C / 2 < kRecords ? C / 2 : kRecords) / kStep;

// The recorded part of the count pass.  A wave whose lanes all hold whole
// chunks (wave_full) takes its sure steps unmasked (no activity tests);
// lastex is then the last sure lookup until a masked step finds a later one.
template <int C, int TB, bool kShort>
__device__ __forceinline__ void count_recorded(const char* s_stream_b, const uint32_t* s_tx, uint32_t col_addr, int cd,
                                               uint32_t rend, bool wave_full, uint32_t& r, uint32_t& cnt4,
                                               uint32_t& lastex, bool& act, int& nq, uint32_t (&rec)[kRecords])
{
    constexpr int U = kSureSteps<C>;
    if (U > 0 && wave_full) {
        count_steps<TB, 0, U, false, kShort>(s_stream_b, s_tx, col_addr, cd, rend, r, cnt4, lastex, act, nq, rec);
        // the last sure record is a pair's second: take back its own count
        constexpr int kLast = (U > 0 ? U : 1) * kStep - 1;
        lastex = rec[kLast] - (rec[kLast - 1] & 0xFFu);
        act = r > rend;
    } else {
        count_steps<TB, 0, U, true, kShort>(s_stream_b, s_tx, col_addr, cd, rend, r, cnt4, lastex, act, nq, rec);
    }
    count_steps<TB, U, kRecords / kStep, true, kShort>(s_stream_b, s_tx, col_addr, cd, rend, r, cnt4, lastex, act,
                                                       nq, rec);
}

// The decode pass over the recorded entries, two at a time, for the nq steps
// the count pass took (compile-time unrolled like count_steps).
template <int Q>
__device__ __forceinline__ uint32_t emit_steps(uint32_t* s_out, uint32_t ob, int nq, const uint32_t (&rec)[kRecords],
                                               uint32_t& carry)
{
    if constexpr (Q < kRecords / kStep) {
        if (Q >= nq) return ob;
#pragma unroll
        for (int j = 0; j < kStep; j += 2)
            ob = emit_pair(s_out, ob, rec[kStep * Q + j], rec[kStep * Q + j + 1], carry);
        return emit_steps<Q + 1>(s_out, ob, nq, rec, carry);
    }
    return ob;
}

// LDS of one decode workgroup, in dwords: decode table | nibble staging |
// stream rows | wave sums.  For the tuned shape (C = 16) the stream rows are
// the first dwords of the staging (the rows are read only by the count pass,
// the staging written only after the scan), which keeps 6 workgroups on a
// compute unit.  For other chunk sizes the rows have their own memory, so
// that lanes with more lookups than records can walk the rest from LDS.
template <int C, int TB>
struct DecodeLds {
    static constexpr int kSlot = C / 4 + 1;                                   // dwords per lane: chunk + look-ahead
    static constexpr int kStreamDw = TB * (kSlot + 1);                        // rows, + one row only read at shift 0
    static constexpr int kOutDw = ((8 * C * TB + 15 + 8 + 16) / 8 + 2 + 3) / 4 * 4;   // nibble staging
    static constexpr bool kShared = C == kChunk;                              // rows inside the staging
    static constexpr int kUnionDw = kShared ? (kOutDw > kStreamDw ? kOutDw : kStreamDw) : kOutDw;
    static constexpr int kRowsOff = (int)kTabStride + (kShared ? 0 : kUnionDw);
    static constexpr int kSumOff = (int)kTabStride + kUnionDw + (kShared ? 0 : (kStreamDw + 3) / 4 * 4);
    static constexpr int kDw = kSumOff + TB / 64;
    static_assert(kUnionDw % 4 == 0, "cleared as 16-byte words");
    static_assert(kShared || C == 4 || C == 8 || C % 16 == 0, "chunk loads of 4, 8 or a multiple of 16 bytes");
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
template <int C>
struct BlockIn {
    uint32_t sv[C / 4];   // the lane's C stream bytes (little-endian words)
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

template <int C, int TB>
__device__ __forceinline__ void load_block(const NextTensor& nt, uint64_t gblk, int tid, BlockIn<C>& in)
{
    const uint64_t b = gblk - nt.begin;
    // block offsets first: they are the first of these loads to be needed
    const uint2 o = bld2(make_rsrc(nt.blk_off + b, 16), (tid & 1) * 8u);
    in.off = ((uint64_t)o.y << 32) | o.x;
    // the block's chunks and the look-ahead word of its last lane (the stream
    // has 16 bytes past its last block)
    const Rsrc rs = make_rsrc(nt.stream + b * ((uint64_t)TB * C), (uint64_t)TB * C + 16);
    if constexpr (C % 16 == 0) {
#pragma unroll
        for (int k = 0; k < C / 16; ++k) {
            const uint4 v = bld4(rs, tid * C + 16 * k);
            in.sv[4 * k] = v.x;
            in.sv[4 * k + 1] = v.y;
            in.sv[4 * k + 2] = v.z;
            in.sv[4 * k + 3] = v.w;
        }
    } else if constexpr (C == 8) {
        const uint2 v = bld2(rs, tid * C);
        in.sv[0] = v.x;
        in.sv[1] = v.y;
    } else {
        in.sv[0] = bld(rs, tid * C);
    }
    in.la = bld(rs, tid * C + C);
    in.gb = bld1(make_rsrc(nt.gaps + b * (TB / 2), TB / 2), tid >> 1);
}

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// ------------------------------------------------------------ decode table
// Builds tensor d's packed table in LDS from its code lengths (ECF8 blog
// §3.1.2 table-driven decode; the codes are canonical, so the lengths fix
// them).  Canonical codes in (length, symbol) order occupy consecutive,
// size-aligned ranges of the left-justified 16-bit code space; d->start holds
// each symbol's first code, summed from the lengths when the plan was
// prepared.  Entries:
//   bits  7..0   4 * symbols decoded (0..16): the nibble count of the entry's
//                output, also usable directly as a shift amount (bits 4..0)
//   bits 15..8   bits consumed (1..16)
//   bits 31..16  the symbols as nibbles, first symbol in bits 19..16.
// Entry w < p_long (an 11-bit window whose first codeword has at most kWin
// bits) decodes greedily the whole codewords inside the window, at most
// kMaxSymPerEntry; entry i in [p_long, entries) stands for the 16-bit value
// i + cdelta (a codeword longer than kWin bits, or no codeword of an
// incomplete code, which consumes one bit and decodes nothing).
// Steps: (1) each short symbol's window range is scattered into a
// first-symbol table F (one 16-bit word per 11-bit window: length | symbol
// << 8; windows of no short codeword get length 16, which never fits), at
// most one store per lane and symbol; (2) each lane chains F over its windows
// (the next codeword starts at the window shifted by the bits consumed so
// far); (3) after a barrier, since F shares the table area, the entries are
// stored, and the long region is searched directly.  Called by every lane of
// a workgroup of kBuildThreads lanes (it holds barriers); a barrier of the
// caller orders the stores before any read of the table.
// The decode kernel's LDS copy of a table fills at most kTableMax entries of
// the table area (16 bytes at a time); its last dword holds the published
// claim of the claimed block order.
constexpr int kClaimSlot = (int)kTabStride - 1;
static_assert((kTableMax + 3) / 4 * 4 <= kClaimSlot, "claim slot past every table");
constexpr int kFirstOff = (int)kTabStride - (1 << kWin) / 2;   // F: the last 1024 dwords of the table area
static_assert(kFirstOff >= 0 && kFirstOff % 4 == 0, "first-symbol table inside the table area");
constexpr int kBuildThreads = 256;

__device__ __forceinline__ void build_table(const DevDesc* __restrict__ d, uint32_t* s_tx, int tid)
{
    constexpr int TB = kBuildThreads;
    constexpr int kPer = (1 << kWin) / TB;                  // windows per lane
    static_assert(kPer * TB == (1 << kWin), "windows split evenly over the lanes");
    static_assert(TB >= 64, "the first wave holds a lane per window of the 9..kWin-bit codes");
    const uint32_t* lp = reinterpret_cast<const uint32_t*>(d->len);
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(d->start);
    uint32_t lw[4], sw[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) lw[i] = __builtin_amdgcn_readfirstlane(gld(lp + i));
#pragma unroll
    for (int i = 0; i < 8; ++i) sw[i] = __builtin_amdgcn_readfirstlane(gld(sp + i));
    const uint32_t p_long = __builtin_amdgcn_readfirstlane(gld(&d->p_long));
    auto len_of = [&](int u) -> uint32_t { return (lw[u >> 2] >> (8 * (u & 3))) & 0xFFu; };
    auto start_of = [&](int u) -> uint32_t { return (sw[u >> 1] >> (16 * (u & 1))) & 0xFFFFu; };

    // (1) symbol s of length l <= kWin covers the 2^(kWin - l) windows from
    // its first one.  Lengths 1..8 cover whole groups of 8 windows, at most
    // 256 groups in all: the lane of a group finds the symbol covering it
    // (ranges are disjoint) and stores the group in one 16-byte store.
    // Lengths 9..kWin cover 4, 2 or 1 windows: lane 4 s + j of the first wave
    // stores window j of symbol s.
    uint16_t* const F = reinterpret_cast<uint16_t*>(s_tx + kFirstOff);
    const uint32_t t = (uint32_t)tid;
#pragma unroll
    for (int g0 = 0; g0 < (1 << (kWin - 3)); g0 += TB) {
        const uint32_t w = 8u * (t + (uint32_t)g0);
        uint32_t v = 0;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const uint32_t ls = len_of(s);
            const uint32_t span = ls - 1u < 8u ? 1u << (kWin - ls) : 0u;
            v = w - (start_of(s) >> (16 - kWin)) < span ? ls | ((uint32_t)s << 8) : v;
        }
        if (v) {   // (no range reaches past window 2^kWin - 1)
            const uint32_t v2 = v | (v << 16);
            *reinterpret_cast<uint4*>(F + w) = make_uint4(v2, v2, v2, v2);
        }
    }
    if (t < 64) {
        const uint32_t s = t >> 2, j = t & 3;
        const uint32_t lq = s < 8 ? (s < 4 ? lw[0] : lw[1]) : (s < 12 ? lw[2] : lw[3]);
        const uint32_t ls = (lq >> (8 * (s & 3))) & 0xFFu;
        const uint32_t sq = s < 8 ? (s < 4 ? (s < 2 ? sw[0] : sw[1]) : (s < 6 ? sw[2] : sw[3]))
                                  : (s < 12 ? (s < 10 ? sw[4] : sw[5]) : (s < 14 ? sw[6] : sw[7]));
        const uint32_t st = (sq >> (16 * (s & 1))) & 0xFFFFu;
        if (ls - 9u < (uint32_t)kWin - 8u && j < (1u << (kWin - ls)))
            F[(st >> (16 - kWin)) + j] = (uint16_t)(ls | (s << 8));
    }
    if (p_long < (1u << kWin))
        for (uint32_t w = p_long + t; w < (1u << kWin); w += TB) F[w] = (uint16_t)16u;
    __syncthreads();

    // (2) the short entries, chained over F
    uint32_t ent[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const uint32_t w = t + (uint32_t)(TB * k);
        const uint32_t f1 = F[w];
        const uint32_t c1 = f1 & 0xFFu;
        const uint32_t f2 = F[(w << (c1 & 31)) & 0x7FFu];
        const uint32_t c2 = c1 + (f2 & 0xFFu);
        const uint32_t f3 = F[(w << (c2 & 31)) & 0x7FFu];
        const uint32_t c3 = c2 + (f3 & 0xFFu);
        const uint32_t f4 = F[(w << (c3 & 31)) & 0x7FFu];
        const uint32_t c4 = c3 + (f4 & 0xFFu);
        // lengths are >= 1, so c2 < c3 < c4: the kept symbols are a prefix
        const bool k2 = c2 <= (uint32_t)kWin, k3 = c3 <= (uint32_t)kWin, k4 = c4 <= (uint32_t)kWin;
        const uint32_t n4 = k4 ? 16u : k3 ? 12u : k2 ? 8u : 4u;      // 4 * symbols
        const uint32_t bits = k4 ? c4 : k3 ? c3 : k2 ? c2 : c1;
        const uint32_t sy = (f1 >> 8) | ((f2 >> 4) & 0xF0u) | (f3 & 0xF00u) | ((f4 << 4) & 0xF000u);
        const uint32_t keep = (1u << n4) - 1u;
        ent[k] = n4 | (bits << 8) | ((sy & keep) << 16);
    }
    __syncthreads();

    // (3) store; the long region from the canonical ranges directly
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const uint32_t w = t + (uint32_t)(TB * k);
        if (w < p_long) s_tx[w] = ent[k];
    }
    {
        const uint32_t ne = __builtin_amdgcn_readfirstlane(gld(&d->entries));
        const uint32_t cd = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)gld(&d->cdelta));
        for (uint32_t i = p_long + t; i < ne; i += TB) {
            const uint32_t v = i + cd;
            uint32_t pos = 0, ns = 0, sy = 0;
            while (ns < (uint32_t)kMaxSymPerEntry && pos < 16u) {
                const uint32_t x = (v << pos) & 0xFFFFu;
                uint32_t fl = 0, fs = 0;
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const uint32_t lu = len_of(u);
                    const uint32_t span = lu ? 1u << (16 - lu) : 0u;
                    const bool in = x - start_of(u) < span;
                    fl = in ? lu : fl;
                    fs = in ? (uint32_t)u : fs;
                }
                if (fl == 0 || pos + fl > 16u) break;
                sy |= fs << (4 * ns);
                ns++;
                pos += fl;
            }
            s_tx[i] = (4 * ns) | ((pos ? pos : 1u) << 8) | (sy << 16);
        }
    }
}

// One workgroup per tensor builds its table in LDS (the general form, valid
// for both index forms) and writes it to the workspace, once per plan: the
// codebooks are fixed, and each decode workgroup copies the table of the
// tensor it works on into its LDS (a 9 KB copy from L2 costs a decode
// workgroup less than the build, whose chained LDS reads conflict).
__global__ __launch_bounds__(kBuildThreads) void ecf8_table_kernel(const DevDesc* __restrict__ descs,
                                                                    uint32_t* __restrict__ tables)
{
    __shared__ __align__(16) uint32_t s_tab[kTabStride];
    const DevDesc* d = descs + blockIdx.x;
    build_table(d, s_tab, (int)threadIdx.x);
    __syncthreads();
    const uint32_t n4 = (gld(&d->entries) + 3) / 4;
    uint4* dst = reinterpret_cast<uint4*>(tables + (uint64_t)blockIdx.x * kTabStride);
    for (uint32_t i = threadIdx.x; i < n4; i += kBuildThreads) dst[i] = reinterpret_cast<const uint4*>(s_tab)[i];
}

#ifndef ECF8_MIN_WAVES
#define ECF8_MIN_WAVES 6
#endif

// Waves per SIMD the register allocation aims for: ECF8_MIN_WAVES, or fewer
// where the workgroup's LDS already allows fewer (160 KB per compute unit).
template <int C, int TB>
constexpr int kWavesTarget = [] {
    const int wgs = 160 * 1024 / (DecodeLds<C, TB>::kDw * 4);
    const int w = wgs * (TB / 64) / 4;
    return w < 1 ? 1 : (w < ECF8_MIN_WAVES ? w : ECF8_MIN_WAVES);
}();

// kShort: every tensor's code is complete with no codeword longer than kWin
// bits (the host launches this form only then; a tensor whose table says
// otherwise is not decoded and its blocks are counted as bad).
// kClaim: the block order.  false: workgroup g takes blocks g, g + G, g + 2G,
// ... (G workgroups).  true: blocks are taken in claims of `claim`
// consecutive blocks; workgroup g's first claim is [g * claim, (g + 1) *
// claim), and every later one comes from a counter in sched[0] (claims
// continue from G * claim), requested one claim ahead.  Over a long dispatch
// the static order lets the workgroups drift apart, spreading the blocks in
// flight over a growing address range; claims keep them within a window of
// about G * claim blocks.  The last workgroup to finish (sched[1] counts
// them) resets both counters, so every run starts from zero.
template <int C, int TB, bool kShort, bool kClaim>
__global__ __launch_bounds__(TB) __attribute__((amdgpu_waves_per_eu(kWavesTarget<C, TB>))) void ecf8_decode_kernel(const DevDesc* __restrict__ descs, int count,
                                                         uint64_t total_blocks,
                                                         const uint32_t* __restrict__ tables,
                                                         unsigned long long* __restrict__ status,
                                                         unsigned int* __restrict__ sched, uint32_t claim)
{
    using L = DecodeLds<C, TB>;
    constexpr int kWaves = TB / 64;
    constexpr int S = L::kSlot;
    constexpr uint32_t R0 = 32u * (S + 1);     // r = R0 - bit position in the lane's chunk
    // One LDS arena: decode table | nibble staging | (stream rows) | wave
    // sums.  For C = 16 the first S * TB dwords of the staging double as the
    // stream rows: they are read only by the count pass and the staging is
    // written only after the block-wide scan, so a lane clears its own rows
    // once it has counted, the write-back clears what the decode wrote, and a
    // barrier at the top of each block orders the previous block's write-back
    // before the new rows are written.
    constexpr int kUnionOff = (int)kTabStride;
    __shared__ __align__(256) uint32_t lds[L::kDw];
    uint32_t* const s_tx = lds;
    uint32_t* const s_out = lds + kUnionOff;
    uint32_t* const s_stream = lds + L::kRowsOff;
    uint32_t* const s_wsum = lds + L::kSumOff;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // Lane words in word-major, reversed order: word k of the lane's chunk
    // (k = 0..S-1, k = S-1 the look-ahead) lives in row S - k, element tid;
    // row S + 1 (staging memory) is only read with a zero funnel shift, and a
    // finished lane may read row 0 (dwords before the rows) for a window it
    // drops.  With r = R0 - bitpos, the window pair (word ceil(bitpos/32)-1,
    // next word) is rows (r >> 5) and (r >> 5) - 1, and the funnel shift is
    // r & 31.
    uint32_t* const col = s_stream - TB + tid;                 // col[row * TB] = row `row`, rows 1..S+1
    const uint32_t col_addr = (uint32_t)tid * 4u;              // byte address of row 1, this lane
    const char* const s_stream_b = reinterpret_cast<const char*>(s_stream);

    // claimed order: the end of the claim being decoded, the first block of the
    // next one (known once published), and (lane 0 of the workgroup) the
    // counter value its request returned
    uint64_t c_end = 0, n_base = 0;
    uint32_t pend = 0;
    int req_in = -1;                   // iterations until the pending request is issued (-1: none)
    auto claim_exit = [&]() {
        if (tid == 0 && atomicAdd(&sched[1], 1u) == gridDim.x - 1u) {
            atomicExch(&sched[0], 0u);
            atomicExch(&sched[1], 0u);
        }
    };
    uint64_t blk = blockIdx.x;
    if constexpr (kClaim) {
        blk = (uint64_t)blockIdx.x * claim;
        c_end = blk + claim < total_blocks ? blk + claim : total_blocks;
        if (blk >= total_blocks) {
            claim_exit();
            return;
        }
    }
    if (blk >= total_blocks) return;
    for (int i = tid; i < L::kUnionDw / 4; i += TB) reinterpret_cast<uint4*>(s_out)[i] = make_uint4(0, 0, 0, 0);

    NextTensor nt;
    fetch_next_tensor(descs, 0, nt);
    while (nt.t + 1 < count && blk >= nt.end) fetch_next_tensor(descs, nt.t + 1, nt);
    BlockIn<C> nx;
    load_block<C, TB>(nt, blk, tid, nx);
    int ptens = nt.t;                  // tensor of the prefetched block
    const uint32_t cap = 8u * C * TB;  // staging capacity in elements

    // fields of the tensor being decoded
    int cur = -1;
    uint64_t c_begin = 0, c_n = 0, c_T = 0, c_lenpack = 0;
    const uint8_t* c_nib = nullptr;
    const uint8_t* c_stream = nullptr;
    uint8_t* c_out = nullptr;
    int c_cd = 0;
    uint32_t c_ok = 0;
    // Takes tensor t's fields and copies its decode table into LDS: 16-byte
    // loads, at most 3 per lane (each load waits for every memory operation in
    // flight, the previous block's stores too, so fewer, wider loads cost fewer
    // round trips: 3% faster than dword loads).
    auto take_tensor = [&](int t) {
        const DevDesc* d = descs + t;
        c_begin = d->block_begin;
        c_n = d->n;
        c_T = d->total_bits;
        c_lenpack = d->lenpack;
        c_nib = d->nibbles;
        c_stream = d->stream;
        c_out = d->out;
        c_cd = d->cdelta;
        c_ok = !kShort || c_cd == kShortCd;   // 0: a code the short form cannot index
        const uint32_t n4 = (d->entries + 3) / 4;
        const Rsrc rt = make_rsrc(tables + (uint64_t)t * kTabStride, 16ull * n4);
        for (uint32_t i = tid; i < n4; i += TB)
            reinterpret_cast<u32x4*>(s_tx)[i] = __builtin_amdgcn_raw_buffer_load_b128(rt, 16u * i, 0, 0);
        cur = t;
    };
    // the first tensor's table is requested together with the first block's
    // inputs, so the two latencies overlap
    take_tensor(ptens);
    // wait for the first block's loads here, so that at the loop head only the
    // back edge has loads in flight and the compiler can count them exactly
    asm volatile("" ::"v"(nx.sv[0]), "v"(nx.la), "v"(nx.gb), "v"((uint32_t)nx.off));
    // The request for the claim after the first is needed on the first claim's
    // second-to-last block; the workgroups issue it on different blocks before
    // that, so that they do not all queue on the counter at once.  (A request
    // is issued after its iteration's loads: a wait for those loads then does
    // not wait for it.)
    if constexpr (kClaim)
        if (c_end < total_blocks) req_in = claim > 2 ? (int)(blockIdx.x % (claim - 2)) : 0;

    uint64_t nb = 0;                   // the block prefetched for the next iteration
    for (; blk < total_blocks; blk = nb) {
        const BlockIn<C> in = nx;
        const uint64_t blk_end = c_end;    // end of the claim holding blk
        // (every lane left the previous decode pass at its closing barrier, so
        // the old table is no longer read)
        if (ptens != cur) take_tensor(ptens);
        // the table is in place and every lane has finished the previous block's
        // write-back, whose staging memory the stream rows reuse
        __syncthreads();
        // stage the chunk (big-endian words, reversed order) into the lane's rows
#pragma unroll
        for (int k = 0; k < C / 4; ++k) col[(S - k) * TB] = __builtin_bswap32(in.sv[k]);
        col[TB] = __builtin_bswap32(in.la);                   // row 1: the look-ahead word
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
        if constexpr (kClaim) {
            if (blk + 1 < c_end) {
                nb = blk + 1;
            } else if (c_end < total_blocks) {
                // the next claim (published a block ago); request the one after it
                nb = n_base;
                c_end = n_base + claim < total_blocks ? n_base + claim : total_blocks;
                if (c_end < total_blocks) req_in = 0;
            } else {
                nb = total_blocks;
            }
        } else {
            nb = blk + gridDim.x;
        }
        const uint64_t nbe = nb < total_blocks ? nb : blk;
        while (nt.t + 1 < count && nbe >= nt.end) fetch_next_tensor(descs, nt.t + 1, nt);
        load_block<C, TB>(nt, nbe, tid, nx);
        ptens = nt.t;
        if constexpr (kClaim) {
            if (req_in == 0 && tid == 0) pend = atomicAdd(&sched[0], claim);
            if (req_in >= 0) --req_in;
        }

        // Wave priorities rise through the block: count 1, scan and decode 2,
        // write-back 3, then 0 until the next count.  Among the waves of a SIMD
        // (each from another workgroup, at another point of its block), the one
        // nearest its stores issues first, so stores leave earlier and the
        // next blocks' loads start sooner (4% faster than one raised count).
        __builtin_amdgcn_s_setprio(1);
        // ---- phase 2: count the codewords that start inside [gap, E)
        // The walk runs in steps of kStep lookups with one wave-uniform exit test
        // per step; a lane that has passed E keeps looking up at its final
        // position but records 0 (no bits, no symbols).  The recorded entries sit
        // in statically indexed registers and are replayed by phase 4, so the
        // stream is walked once (lanes with more than kRecords lookups finish with
        // a plain walk).
        const int cd = c_cd;
        const uint32_t rend = R0 - E;
        const uint32_t r0 = R0 - gap;
        uint32_t rec[kRecords];
        uint32_t r = r0;
        uint32_t cnt4 = 0, lastex = 0;
        bool act = r > rend;
        int nq = 0;                        // steps taken (wave-uniform)
        const bool wave_full = leftc >= 8u * C * 64u * (uint32_t)(wave + 1);
        count_recorded<C, TB, kShort>(s_stream_b, s_tx, col_addr, cd, rend, wave_full, r, cnt4, lastex, act, nq, rec);
        const uint32_t r_rec = r;          // where the recorded lookups end
        while (r > rend) {
            const uint32_t e = lookup<TB>(s_stream_b, s_tx, col_addr, r, cd);
            lastex = e;
            r -= (e >> 8) & 0xFFu;
            cnt4 += e & 0xFFu;
        }
        __builtin_amdgcn_s_setprio(2);
        if constexpr (L::kShared) {
            // the lane's rows are staging memory from here on: leave them cleared
#pragma unroll
            for (int k = 0; k < S; ++k) col[(S - k) * TB] = 0u;
        }
        uint32_t cnt = cnt4 >> 2;
        if (r != r0) {
            // the last lookup (at r + its bit count) may have decoded codewords
            // that start at or after E: keep those starting before E
            const uint32_t ex = lastex;
            const uint32_t ns = (ex & 0xFFu) >> 2;
            const uint32_t room = r + ((ex >> 8) & 0xFFu) - rend;
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
        asm volatile("" ::"v"(nx.sv[0]), "v"(nx.la), "v"(nx.gb), "v"((uint32_t)nx.off));
        // claimed order: on the claim's second-to-last block, lane 0 publishes
        // the next claim's start (its request went out at least a block ago,
        // before the loads just waited for, unless a claim is 2 blocks), and
        // every lane reads it after the barrier
        const bool publish = kClaim && blk + 2 == blk_end && blk_end < total_blocks;
        if (publish && tid == 0) lds[kClaimSlot] = pend;

        // ---- phase 3: block-wide exclusive scan of the counts
        const uint32_t incl = wave_inclusive_scan(cnt);
        if (lane == 63) s_wsum[wave] = incl;
        __syncthreads();
        if (publish)
            n_base = (uint64_t)gridDim.x * claim + (uint32_t)__builtin_amdgcn_readfirstlane((int)lds[kClaimSlot]);
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
        uint32_t carry = 0;
        ob = emit_steps<0>(s_out, ob, nq, rec, carry);
        // the last pair's spill belongs to the dword after the one ob was in
        // before that pair; that is the dword of ob or the one before it, and
        // ob's dword when the spill is non-zero (a spill means the pair crossed)
        if (nq) atomicOr(&s_out[ob >> 5], carry);
        if (r_rec > rend) {
            // lanes with more than kRecords lookups walk the rest
            r = r_rec;
            if constexpr (L::kShared) {
                // their rows are staging memory now: reload the chunk (L2-resident)
                // into registers and take windows from there
                const uint8_t* sp = c_stream + (b * TB + tid) * C;
                const uint4 cv = gld4(sp);
                const uint32_t w[5] = {__builtin_bswap32(cv.x), __builtin_bswap32(cv.y), __builtin_bswap32(cv.z),
                                       __builtin_bswap32(cv.w),
                                       __builtin_bswap32(gld(reinterpret_cast<const uint32_t*>(sp + C)))};
                while (r > rend) {
                    const uint32_t win = reg_window(w, R0 - r);
                    const uint32_t ex = s_tx[table_index(win, cd)];
                    emit_symbols(s_out, ob, ex);
                    ob += ex & 0xFFu;
                    r -= (ex >> 8) & 0xFFu;
                }
            } else {
                // their rows are intact: take windows from LDS
                while (r > rend) {
                    const uint32_t ex = lookup<TB>(s_stream_b, s_tx, col_addr, r, cd);
                    emit_symbols(s_out, ob, ex);
                    ob += ex & 0xFFu;
                    r -= (ex >> 8) & 0xFFu;
                }
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
        // whole groups of the prefetched range, one store each (group 0 of a
        // block that starts mid-group is an edge, written below)
#pragma unroll
        for (int k = 0; k < kNibPrefetch; ++k) {
            const uint32_t g = tid + k * TB;
            if (g >= end_full) break;
            if (g >= first_full) write_full(s_out, out_blk, g, nv[k]);
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
        // The write-back read and cleared groups [0, groups).  The decode wrote
        // groups [0, zend), the codewords a last lane decodes past the end
        // included (and more or fewer when a corrupt block's count is off):
        // clear the rest (groups no lane read; the next block writes the
        // staging only after its barriers).
        {
            const uint32_t zend0 = (a0 + total + 3u + 15u) >> 4;
            const uint32_t zend = zend0 < (uint32_t)(L::kOutDw / 2) ? zend0 : (uint32_t)(L::kOutDw / 2);
            for (uint32_t g = groups + tid; g < zend; g += TB)
                reinterpret_cast<uint2*>(s_out)[g] = make_uint2(0u, 0u);
        }
    }
    if constexpr (kClaim) claim_exit();
}

// ------------------------------------------------------------ host helpers
// The (C, TB) shapes with a decode kernel.  (16, 256) is the tuned one; the
// others decode the same format with the same steps (the pages' own 64-byte
// chunks on 128 lanes among them).
#define ECF8_DECODE_SHAPES(X) X(16, 256) X(32, 256) X(64, 128) X(16, 128) X(8, 256) X(16, 512)

// Index of a supported shape, or -1.
int shape_index(uint32_t C, uint32_t TB)
{
    int i = 0;
#define ECF8_X(c, t) \
    if (C == (c) && TB == (t)) return i; \
    ++i;
    ECF8_DECODE_SHAPES(ECF8_X)
#undef ECF8_X
    return -1;
}

const void* decode_kernel_ptr(int shape, bool short_codes)
{
    int i = 0;
#define ECF8_X(c, t)                                                                                         \
    if (shape == i)                                                                                          \
        return short_codes ? reinterpret_cast<const void*>(ecf8_decode_kernel<c, t, true, false>)            \
                           : reinterpret_cast<const void*>(ecf8_decode_kernel<c, t, false, false>);          \
    ++i;
    ECF8_DECODE_SHAPES(ECF8_X)
#undef ECF8_X
    return nullptr;
}

// The decode dispatch; with events, they are attached to the dispatch itself
// and take its start and end times.
// claim > 0: the claimed block order with claims of that many blocks (sched:
// the two zeroed counters); 0: the static order (sched unused).
int launch_decode(uint32_t C, uint32_t TB, bool short_codes, uint32_t grid, hipStream_t st, const DevDesc* dd,
                  int count, uint64_t blocks, const uint32_t* tables, unsigned long long* status,
                  unsigned int* sched, uint32_t claim, hipEvent_t start = nullptr, hipEvent_t stop = nullptr)
{
#define ECF8_LAUNCH(k)                                                                                        \
    do {                                                                                                      \
        if (start || stop)                                                                                    \
            hipExtLaunchKernelGGL((k), dim3(grid), dim3(TB), 0, st, start, stop, 0, dd, count, blocks, tables, \
                                  status, sched, claim);                                                      \
        else                                                                                                  \
            hipLaunchKernelGGL((k), dim3(grid), dim3(TB), 0, st, dd, count, blocks, tables, status, sched,     \
                               claim);                                                                        \
    } while (0)
#define ECF8_X(c, t)                                                                                          \
    if (C == (c) && TB == (t)) {                                                                              \
        if (short_codes && claim)                                                                             \
            ECF8_LAUNCH((ecf8_decode_kernel<c, t, true, true>));                                              \
        else if (short_codes)                                                                                 \
            ECF8_LAUNCH((ecf8_decode_kernel<c, t, true, false>));                                             \
        else if (claim)                                                                                       \
            ECF8_LAUNCH((ecf8_decode_kernel<c, t, false, true>));                                             \
        else                                                                                                  \
            ECF8_LAUNCH((ecf8_decode_kernel<c, t, false, false>));                                            \
        return hipGetLastError() == hipSuccess ? ECF8_OK : ECF8_ERR_HIP;                                      \
    }
    ECF8_DECODE_SHAPES(ECF8_X)
#undef ECF8_X
#undef ECF8_LAUNCH
    return ECF8_ERR_UNSUPPORTED;
}

// A complete code with no codeword longer than kWin bits: the tables of such
// tensors are indexed by the 11-bit prefix alone (the short kernel form).
bool short_code(const ecf8_codebook& cb)
{
    uint32_t units = 0;                          // 11-bit prefixes covered
    for (int s = 0; s < 16; ++s) {
        const uint32_t l = cb.len[s];
        if (l > (uint32_t)kWin) return false;
        if (l) units += 1u << (kWin - l);
    }
    return units == (1u << kWin);
}

constexpr int kShapes = 6;
struct DeviceInfo {
    int cus = 0;
    int occupancy = 0;
};

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices][kShapes][2];   // fixed size: the decode paths allocate no host memory either

int device_info(uint32_t C, uint32_t TB, bool short_codes, DeviceInfo* out)
{
    const int shape = shape_index(C, TB);
    if (shape < 0 || shape >= kShapes) return ECF8_ERR_UNSUPPORTED;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ECF8_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return ECF8_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DeviceInfo& di = g_dev[dev][shape][short_codes ? 1 : 0];
    if (di.cus == 0) {
        int cus = 0, occ = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return ECF8_ERR_HIP;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, decode_kernel_ptr(shape, short_codes), (int)TB, 0) !=
            hipSuccess)
            return ECF8_ERR_HIP;
        di.cus = cus > 0 ? cus : 1;
        di.occupancy = occ > 0 ? occ : 1;
    }
    *out = di;
    return ECF8_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Validates one tensor of a batch and writes its device descriptor (host
// memory, copied to the device by the caller); `blocks` is the running block
// count of the batch.
int fill_desc(const ecf8_tensor_desc& td, uint8_t* out_base, uint64_t& blocks, DevDesc& dd)
{
    const ecf8_meta& m = td.meta;
    int rc = ecf8_validate_meta(&m);
    if (rc) return rc;
    if (shape_index(m.chunk_bytes, m.threads_per_block) < 0) return ECF8_ERR_UNSUPPORTED;
    if (m.n > 0) {
        if (!out_base || !td.s.stream || !td.s.nibbles || !td.s.gaps || !td.s.blk_off) return ECF8_ERR_ARG;
        if (!aligned(td.s.stream, 16) || !aligned(td.s.nibbles, 8) || !aligned(td.s.blk_off, 8) ||
            !aligned(out_base + td.out_offset, 16))
            return ECF8_ERR_ARG;
    }
    std::memset(&dd, 0, sizeof(dd));
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
    // the table's split point: every code of at most kWin bits precedes the
    // long ones, so the first long 11-bit prefix is the short codes' space
    uint32_t short_units = 0;
    for (int s = 0; s < 16; ++s) {
        const uint32_t l = m.cb.len[s];
        if (!l) continue;
        dd.lenpack |= (uint64_t)((l - 1) & 15) << (4 * s);
        if (l <= (uint32_t)kWin) short_units += 1u << (16 - l);
    }
    dd.p_long = short_units >> (16 - kWin);
    for (int s = 0; s < 16; ++s) {
        const uint32_t l = m.cb.len[s];
        uint32_t st = 0;
        for (int u = 0; u < 16 && l; ++u) {
            const uint32_t lu = m.cb.len[u];
            if (lu && (lu < l || (lu == l && u < s))) st += 1u << (16 - lu);
        }
        dd.start[s] = (uint16_t)st;   // < 2^16: the code space before a used symbol is not full
    }
    dd.cdelta = (int32_t)(((1u << (16 - kWin)) - 1) * dd.p_long);
    const uint32_t entries = 65536u - (uint32_t)dd.cdelta;      // <= kTableMax for every complete code
    dd.entries = entries < (uint32_t)kTableMax ? entries : (uint32_t)kTableMax;
    return ECF8_OK;
}

// The (C, TB) all tensors of a batch share: every tensor's own, which must be
// a supported shape and the same for all (ECF8_ERR_UNSUPPORTED otherwise).
// An empty batch takes the tuned shape.
int batch_shape(const ecf8_tensor_desc* descs, int count, uint32_t* C, uint32_t* TB)
{
    *C = kChunk;
    *TB = kLanes;
    for (int i = 0; i < count; ++i) {
        const ecf8_meta& m = descs[i].meta;
        if (i == 0) {
            *C = m.chunk_bytes;
            *TB = m.threads_per_block;
        } else if (m.chunk_bytes != *C || m.threads_per_block != *TB) {
            return ECF8_ERR_UNSUPPORTED;
        }
    }
    return shape_index(*C, *TB) >= 0 || count == 0 ? ECF8_OK : ECF8_ERR_UNSUPPORTED;
}

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
    std::vector<unsigned char> host(table_offset(count), 0);   // cleared status + descriptors
    DevDesc* hd = reinterpret_cast<DevDesc*>(host.data() + desc_offset());
    uint64_t blocks = 0;
    uint32_t C = kChunk, TB = kLanes;
    int rc = batch_shape(descs, count, &C, &TB);
    if (rc) return rc;
    bool short_codes = true;
    for (int i = 0; i < count; ++i) {
        rc = fill_desc(descs[i], out_base, blocks, hd[i]);
        if (rc) return rc;
        short_codes = short_codes && short_code(descs[i].meta.cb);
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (hipMemcpyAsync(workspace, host.data(), host.size(), hipMemcpyHostToDevice, st) != hipSuccess)
        return ECF8_ERR_HIP;
    if (count > 0) {
        // each tensor's decode table, once per plan (the codebooks are fixed)
        unsigned char* ws = static_cast<unsigned char*>(workspace);
        hipLaunchKernelGGL(ecf8_table_kernel, dim3(count), dim3(kBuildThreads), 0, st,
                           reinterpret_cast<const DevDesc*>(ws + desc_offset()),
                           reinterpret_cast<uint32_t*>(ws + table_offset(count)));
        if (hipGetLastError() != hipSuccess) return ECF8_ERR_HIP;
    }
    DeviceInfo di;
    rc = device_info(C, TB, short_codes, &di);
    if (rc) return rc;
    uint64_t grid = (uint64_t)di.cus * (uint64_t)di.occupancy;
    if (grid > blocks) grid = blocks;
    plan->workspace = workspace;
    plan->workspace_bytes = workspace_bytes;
    plan->total_blocks = blocks;
    plan->count = (uint32_t)count;
    plan->chunk_bytes = C;
    plan->threads_per_block = TB;
    plan->grid = (uint32_t)grid;
    plan->short_codes = short_codes ? 1u : 0u;
    plan->claim_blocks = blocks >= kClaimMinBlocksPerWg * grid ? kClaimBlocks : 0u;
    return ECF8_OK;
}

namespace {

int check_plan(const ecf8_plan* plan)
{
    if (!plan) return ECF8_ERR_ARG;
    if (plan->count == 0 || plan->total_blocks == 0) return ECF8_OK;
    if (!plan->workspace || plan->workspace_bytes < ecf8_workspace_bytes((int)plan->count))
        return ECF8_ERR_WORKSPACE;
    if (shape_index(plan->chunk_bytes, plan->threads_per_block) < 0 || plan->grid == 0) return ECF8_ERR_ARG;
    if (plan->claim_blocks) {
        // the counter is 32 bits: it never passes total_blocks + grid * claim_blocks
        if (plan->claim_blocks < 2 || plan->claim_blocks > kClaimBlocksMax) return ECF8_ERR_ARG;
        if (plan->total_blocks + (uint64_t)plan->grid * plan->claim_blocks >= (1ull << 32)) return ECF8_ERR_ARG;
    }
    return ECF8_OK;
}

}  // namespace

namespace {

int run_plan(const ecf8_plan* plan, void* hip_stream, hipEvent_t start, hipEvent_t stop)
{
    int rc = check_plan(plan);
    if (rc || plan->count == 0 || plan->total_blocks == 0) return rc;
    unsigned char* ws = static_cast<unsigned char*>(plan->workspace);
    DevDesc* dd = reinterpret_cast<DevDesc*>(ws + desc_offset());
    auto* status = reinterpret_cast<unsigned long long*>(ws);
    const uint32_t* tables = reinterpret_cast<const uint32_t*>(ws + table_offset((int)plan->count));
    auto* sched = reinterpret_cast<unsigned int*>(ws + kSchedOffset);
    return launch_decode(plan->chunk_bytes, plan->threads_per_block, plan->short_codes != 0, plan->grid,
                         reinterpret_cast<hipStream_t>(hip_stream), dd, (int)plan->count, plan->total_blocks, tables,
                         status, sched, plan->claim_blocks, start, stop);
}

}  // namespace

extern "C" int ecf8_decode_run(const ecf8_plan* plan, void* hip_stream)
{
    return run_plan(plan, hip_stream, nullptr, nullptr);
}

extern "C" int ecf8_decode_run_timed(const ecf8_plan* plan, void* hip_stream, void* start_event, void* stop_event)
{
    return run_plan(plan, hip_stream, reinterpret_cast<hipEvent_t>(start_event),
                    reinterpret_cast<hipEvent_t>(stop_event));
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
    if (v) {   // restart the count
        const unsigned long long zero = 0;
        if (hipMemcpy(const_cast<void*>(workspace), &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
            return ECF8_ERR_HIP;
    }
    return v ? ECF8_ERR_CORRUPT : ECF8_OK;
}

// ------------------------------------------------------------ no-allocation entry point
// ecf8_decode_batched without a workspace argument, for callers that cannot
// allocate (HIP graph capture, serving loops that forbid allocation): the
// status word, descriptors and decode tables live in `scratch`, a fixed
// device array of this library (one copy per GPU, held until the process
// ends).  The descriptors reach the device as kernel arguments of a small
// setup launch, so the call makes no allocation, no copy and no memset.
namespace {

constexpr int kNoAllocMaxTensors = 16;
constexpr int kSetupDescs = 8;                          // descriptors per setup launch (1 KiB of arguments)
constexpr uint64_t kNoAllocScratchBytes =
    kStatusBytes + (kNoAllocMaxTensors * sizeof(DevDesc) + 255) / 256 * 256 + kNoAllocMaxTensors * kTableBytes;
static_assert(kNoAllocScratchBytes == 150016, "scratch size stated in the header");

struct SetupArgs {
    DevDesc d[kSetupDescs];
};

// Copies n descriptors from the kernel arguments to dst (dwords spread over the lanes)
// and, with clear set, zeroes the block-check counter.
__global__ __launch_bounds__(256) void ecf8_noalloc_setup_kernel(SetupArgs a, int n, DevDesc* __restrict__ dst,
                                                                 unsigned long long* __restrict__ status, int clear)
{
    constexpr int kDw = (int)(sizeof(DevDesc) / 4);
    const int t = threadIdx.x;
    for (int i = t; i < n * kDw; i += 256) reinterpret_cast<uint32_t*>(dst)[i] = reinterpret_cast<const uint32_t*>(a.d)[i];
    if (clear && t == 0) *status = 0ull;
}

struct NoAllocDevice {
    unsigned char* ptr = nullptr;   // device address of this GPU's copy of scratch
    bool ready = false;
};
NoAllocDevice g_noalloc[kMaxDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

// The device address of the current GPU's scratch, resolved once per device
// with that device current (the array's host-side name is not a device address).
int noalloc_scratch(unsigned char** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ECF8_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    NoAllocDevice& d = g_noalloc[dev];
    if (!d.ready) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ECF8_ERR_HIP;
        d.ptr = static_cast<unsigned char*>(p);
        d.ready = true;
    }
    *out = d.ptr;
    return ECF8_OK;
}

}  // namespace

extern "C" int ecf8_decode_batched_noalloc(const ecf8_tensor_desc* descs, int count, uint8_t* out_base,
                                           uint64_t* bad_blocks, void* hip_stream)
{
    if (count < 0 || (count > 0 && !descs)) return ECF8_ERR_ARG;
    if (count > kNoAllocMaxTensors) return ECF8_ERR_WORKSPACE;
    if (bad_blocks && !aligned(bad_blocks, 8)) return ECF8_ERR_ARG;
    DevDesc hd[kNoAllocMaxTensors];
    uint64_t blocks = 0;
    uint32_t C = kChunk, TB = kLanes;
    int rc = batch_shape(descs, count, &C, &TB);
    if (rc) return rc;
    bool short_codes = true;
    for (int i = 0; i < count; ++i) {
        rc = fill_desc(descs[i], out_base, blocks, hd[i]);
        if (rc) return rc;
        short_codes = short_codes && short_code(descs[i].meta.cb);
    }
    unsigned char* ws = nullptr;
    rc = noalloc_scratch(&ws);
    if (rc) return rc;
    DeviceInfo di;
    rc = device_info(C, TB, short_codes, &di);
    if (rc) return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    auto* status = bad_blocks ? reinterpret_cast<unsigned long long*>(bad_blocks)
                              : reinterpret_cast<unsigned long long*>(ws);
    DevDesc* dd = reinterpret_cast<DevDesc*>(ws + desc_offset());
    uint32_t* tables = reinterpret_cast<uint32_t*>(ws + table_offset(count));
    // descriptors (and the cleared counter) first, in launches of kSetupDescs
    for (int c = 0; c < count || c == 0; c += kSetupDescs) {
        SetupArgs a;
        const int nc = count - c < kSetupDescs ? count - c : kSetupDescs;
        for (int k = 0; k < kSetupDescs; ++k) a.d[k] = k < nc ? hd[c + k] : DevDesc{};
        hipLaunchKernelGGL(ecf8_noalloc_setup_kernel, dim3(1), dim3(256), 0, st, a, nc, dd + c, status, c == 0 ? 1 : 0);
        if (count == 0) break;
    }
    if (blocks > 0) {
        hipLaunchKernelGGL(ecf8_table_kernel, dim3(count), dim3(kBuildThreads), 0, st, dd, tables);
        uint64_t grid = (uint64_t)di.cus * (uint64_t)di.occupancy;
        if (grid > blocks) grid = blocks;
        return launch_decode(C, TB, short_codes, (uint32_t)grid, st, dd, count, blocks, tables, status, nullptr, 0u);
    }
    return hipGetLastError() == hipSuccess ? ECF8_OK : ECF8_ERR_HIP;
}
