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
// the plan is prepared):
//   * primary: 1024 entries indexed by the next 10 stream bits.  An entry
//     holds the one or two whole codewords those bits start with (symbols,
//     total bits, length of the first), or, for a prefix of codewords longer
//     than 10 bits, a pointer to a subtable;
//   * subtables: one per such prefix, indexed by the next k bits, k being the
//     longest codeword below the prefix minus 10 (1..6).  A complete code
//     of at most 256 symbols needs at most about 2340 subtable entries (a
//     subtree of depth k holds at least k + 1 codewords), so every table
//     fits in 4096 entries (16 KB of LDS).
// Entry bits: 31 pointer flag; pointer: 15..0 subtable base, 19..16 k;
// symbols: 4..0 total bits, 6..5 count (0 = no codeword), 11..7 length of
// the first, 19..12 first symbol, 27..20 second symbol.
//
// Decode kernel: persistent workgroups of TB lanes walk the global block
// index over all tensors.  Per block each lane loads its 16-byte chunk plus
// 4 bytes of look-ahead, walks it from its gap counting codewords that start
// inside the chunk, the workgroup scans the counts (checked against the
// block offsets), and in rounds of at most 16384 symbols the lanes walk
// again writing each symbol byte into LDS at its scanned position (the stage
// aligned to 16 output elements); the workgroup then assembles whole groups
// of 16 elements from 16 symbol bytes and the raw plane with 16-byte loads
// and stores (byte permutes and masks), the ragged ends one element a lane.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "ecf8v.h"

namespace {

constexpr int kChunk = 16;                 // bytes per lane
constexpr int kChunkBits = 8 * kChunk;
constexpr int kPrimBits = 10;
constexpr int kTabEntries = 4096;
constexpr int kStageSyms = 16384;           // symbols staged per round

// Per-tensor descriptor in the workspace.
struct DescV {
    const uint8_t* stream;
    const uint8_t* raw;
    const uint8_t* gaps;
    const uint64_t* blk_off;
    uint8_t* out;
    uint64_t n;
    uint64_t n_blocks;
    uint64_t first_block;      // global index of the tensor's first block
    uint64_t total_bits;       // T: codewords start only before it
    uint8_t len[ECF8V_MAX_SYM];
};

// Workspace: status (bad-block counter, table-overflow counter) | descriptors
// | one table per tensor, each part 256-byte aligned.
constexpr uint64_t kStatusBytes = 256;
uint64_t desc_offset() { return kStatusBytes; }
uint64_t table_offset(int count) { return desc_offset() + ((uint64_t)count * sizeof(DescV) + 255) / 256 * 256; }

__device__ __forceinline__ uint32_t ld_u32(const uint8_t* p)
{
    return *reinterpret_cast<const uint32_t*>(p);
}

// Canonical decode of the top bits of a `width`-bit value v, trying lengths
// lo..hi: the first length l whose prefix falls inside that length's code
// range.  Returns the symbol and sets *len, or -1.
__device__ __forceinline__ int canon_find(uint32_t v, int width, int lo, int hi, const uint32_t* first,
                                          const uint32_t* cnt, const uint16_t* offs, const uint8_t* sorted, int* len)
{
    for (int l = lo; l <= hi; ++l) {
        const uint32_t c = v >> (width - l);
        if (c - first[l] < cnt[l]) {
            *len = l;
            return sorted[offs[l] + (c - first[l])];
        }
    }
    return -1;
}

// One workgroup (256 lanes) per tensor: canonical codes from the lengths,
// then the primary table and the subtables.
__global__ __launch_bounds__(256) void ecf8v_table_kernel(const DescV* __restrict__ descs, uint32_t* __restrict__ tables,
                                                          unsigned long long* __restrict__ status)
{
    __shared__ uint8_t L[ECF8V_MAX_SYM];
    __shared__ uint8_t sorted[ECF8V_MAX_SYM];
    __shared__ uint32_t first[18], cnt[18];
    __shared__ uint16_t offs[18];
    __shared__ uint8_t dmax[1 << kPrimBits];
    __shared__ uint16_t sub_base[1 << kPrimBits];
    __shared__ uint32_t used;
    const int tid = threadIdx.x;
    const DescV& d = descs[blockIdx.x];
    uint32_t* tab = tables + (uint64_t)blockIdx.x * kTabEntries;
    L[tid] = d.len[tid];
    if (tid < 18) cnt[tid] = 0;
    __syncthreads();
    if (L[tid]) atomicAdd(&cnt[L[tid]], 1u);
    __syncthreads();
    if (tid == 0) {
        uint32_t c = 0, o = 0;
        for (int l = 1; l <= 16; ++l) {
            c = (c + cnt[l - 1]) << 1;
            first[l] = c;
            offs[l] = (uint16_t)o;
            o += cnt[l];
        }
        first[17] = 0;
        cnt[17] = 0;
        offs[17] = (uint16_t)o;
    }
    __syncthreads();
    const int ls = L[tid];
    uint32_t code = 0;
    if (ls) {
        uint32_t rank = 0;
        for (int s = 0; s < tid; ++s) rank += L[s] == ls;
        code = first[ls] + rank;
        sorted[offs[ls] + rank] = (uint8_t)tid;
    }
    __syncthreads();
    // longest codeword below each long prefix
    __shared__ uint32_t dmax32[1 << kPrimBits];
    for (int i = tid; i < (1 << kPrimBits); i += 256) dmax32[i] = 0;
    __syncthreads();
    if (ls > kPrimBits) atomicMax(&dmax32[code >> (ls - kPrimBits)], (uint32_t)ls);
    __syncthreads();
    {
        // subtable bases: an exclusive scan of the subtable sizes, 4 prefixes a lane
        uint32_t sz[4], mine = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t dm = dmax32[4 * tid + q];
            dmax[4 * tid + q] = (uint8_t)(dm ? dm - kPrimBits : 0);
            sz[q] = dm ? 1u << (dm - kPrimBits) : 0u;
            mine += sz[q];
        }
        __shared__ uint32_t part[256];
        part[tid] = mine;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {         // Hillis-Steele inclusive scan
            const uint32_t v = tid >= off ? part[tid - off] : 0u;
            __syncthreads();
            part[tid] += v;
            __syncthreads();
        }
        uint32_t next = (1u << kPrimBits) + part[tid] - mine;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            sub_base[4 * tid + q] = (uint16_t)(next < 65535 ? next : 65535);
            next += sz[q];
        }
        if (tid == 255) {
            used = next;
            if (next > (uint32_t)kTabEntries) atomicAdd(status + 1, 1ull);
        }
    }
    __syncthreads();
    const bool fits = used <= (uint32_t)kTabEntries;
    // primary entries
    for (int i = tid; i < (1 << kPrimBits); i += 256) {
        uint32_t e = 0;
        if (dmax[i] && fits) {
            e = 0x80000000u | ((uint32_t)dmax[i] << 16) | sub_base[i];
        } else {
            int l1 = 0;
            const int s1 = canon_find((uint32_t)i, kPrimBits, 1, kPrimBits, first, cnt, offs, sorted, &l1);
            if (s1 >= 0) {
                e = (uint32_t)l1 | (1u << 5) | ((uint32_t)l1 << 7) | ((uint32_t)s1 << 12);
                const int w2 = kPrimBits - l1;
                if (w2 > 0) {
                    int l2 = 0;
                    const uint32_t rem = (uint32_t)i & ((1u << w2) - 1u);
                    const int s2 = canon_find(rem, w2, 1, w2, first, cnt, offs, sorted, &l2);
                    if (s2 >= 0) e = (uint32_t)(l1 + l2) | (2u << 5) | ((uint32_t)l1 << 7) | ((uint32_t)s1 << 12) |
                                     ((uint32_t)s2 << 20);
                }
            }
        }
        tab[i] = e;
    }
    // subtables
    if (fits) {
        for (int i = tid; i < (1 << kPrimBits); i += 256) {
            const int k = dmax[i];
            if (!k) continue;
            for (int j = 0; j < (1 << k); ++j) {
                const uint32_t v = ((uint32_t)i << k) | (uint32_t)j;
                int l = 0;
                const int s = canon_find(v, kPrimBits + k, kPrimBits + 1, kPrimBits + k, first, cnt, offs, sorted, &l);
                tab[sub_base[i] + j] = s >= 0 ? ((uint32_t)l | (1u << 5) | ((uint32_t)l << 7) | ((uint32_t)s << 12)) : 0u;
            }
        }
    }
}

__global__ __launch_bounds__(64) void ecf8v_clear_kernel(unsigned long long* status, uint32_t words)
{
    if (threadIdx.x < words) status[threadIdx.x] = 0ull;
}

__device__ __forceinline__ uint32_t bswap(uint32_t x) { return __builtin_bswap32(x); }

// Block scan over kTB lanes; returns the exclusive prefix, *total the sum.
template <int kTB>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t x = v;
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);
    const uint32_t r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
                   r2 = __builtin_amdgcn_readlane(x, 47), r3 = __builtin_amdgcn_readlane(x, 63);
    const int row = lane >> 4;
    x += (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
    if (lane == 0) wsum[wave] = r0 + r1 + r2 + r3;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kTB / 64; ++w) {
        before += w < wave ? wsum[w] : 0u;
        all += wsum[w];
    }
    *total = all;
    return before + x - v;
}

// Table lookup at the window; returns the symbols entry (0 = no codeword).
__device__ __forceinline__ uint32_t lookup(const uint32_t* tab, uint32_t tab_n, uint32_t win)
{
    uint32_t e = tab[win >> (32 - kPrimBits)];
    if (e & 0x80000000u) {
        const uint32_t k = (e >> 16) & 15u;
        const uint32_t i = (e & 0xFFFFu) + ((win << kPrimBits) >> (32 - k));
        e = tab[i < tab_n ? i : 0u];
        if (e & 0x80000000u) e = 0;
    }
    return e;      // total bits 0: no codeword
}

template <int kFmt, int kTB>
__global__ __launch_bounds__(256) void ecf8v_decode_kernel(const DescV* __restrict__ descs, int count,
                                                           const uint32_t* __restrict__ tables, uint64_t total_blocks,
                                                           unsigned long long* __restrict__ status, uint32_t tab_n)
{
    // dynamic LDS: the stage (element j at j - (first element & ~15)), then
    // tab_n table entries (the largest table of the plan, a multiple of 4)
    extern __shared__ __align__(16) uint8_t dyn[];
    uint8_t* const stage = dyn;
    uint32_t* const tab = reinterpret_cast<uint32_t*>(dyn + kStageSyms + 32);
    __shared__ uint32_t wsum[kTB / 64];
    const int tid = threadIdx.x;
    int t = -1;
    uint64_t t_first = 0, t_end = 0;
    for (uint64_t gb = blockIdx.x; gb < total_blocks; gb += gridDim.x) {
        if (gb >= t_end) {                                // next tensor(s): blocks come in increasing order
            do {
                ++t;
                t_first = descs[t].first_block;
                t_end = t_first + descs[t].n_blocks;
            } while (gb >= t_end && t + 1 < count);
            __syncthreads();                              // the previous table is no longer read
            const uint4* src = reinterpret_cast<const uint4*>(tables + (uint64_t)t * kTabEntries);
            for (uint32_t i = tid; i < tab_n / 4; i += kTB) reinterpret_cast<uint4*>(tab)[i] = src[i];
            __syncthreads();
        }
        const DescV& d = descs[t];
        const uint64_t lb = gb - t_first;
        const uint64_t blk0 = d.blk_off[lb], blk1 = d.blk_off[lb + 1];
        const uint64_t c = lb * kTB + tid;                // chunk of this lane
        const uint4 v = *reinterpret_cast<const uint4*>(d.stream + c * kChunk);
        const uint32_t W[5] = {bswap(v.x), bswap(v.y), bswap(v.z), bswap(v.w),
                               bswap(ld_u32(d.stream + (c + 1) * kChunk))};
        const uint32_t gap = (d.gaps[c >> 1] >> (4 * (uint32_t)(c & 1))) & 15u;
        // codewords start before the chunk end and before T
        const uint64_t cstart = c * (uint64_t)kChunkBits;
        const uint32_t end = d.total_bits <= cstart ? 0u
                             : (d.total_bits - cstart < (uint64_t)kChunkBits ? (uint32_t)(d.total_bits - cstart)
                                                                            : (uint32_t)kChunkBits);

        // count the codewords that start inside the chunk.  Four phases, one
        // per 32-bit word: a codeword starting in word q lies inside words q
        // and q + 1 (at most 16 bits), so each phase windows a fixed pair.
        // Every symbol of an entry is counted; only the last lookup can hold
        // a second codeword starting at or past the end, taken off after the
        // walk.  A lookup with no codeword moves the position by 256, which
        // ends the walk and marks the chunk bad.
        uint32_t pos = gap, n_here = 0, p_last = 0, e_last = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t lim = end < 32u * (q + 1) ? end : 32u * (q + 1);
            const uint64_t pair = ((uint64_t)W[q] << 32) | W[q + 1];
            while (pos < lim) {
                const uint32_t e = lookup(tab, tab_n, (uint32_t)((pair << (pos - 32u * q)) >> 32));
                const uint32_t nb = e & 31u;
                n_here += (e >> 5) & 3u;
                p_last = pos;
                e_last = e;
                pos += nb ? nb : 256u;
            }
        }
        const bool bad = pos >= 256u;
        if (((e_last >> 5) & 3u) == 2u && p_last + ((e_last >> 7) & 31u) >= end) n_here -= 1;
        uint32_t total;
        const uint32_t off = block_excl_scan<kTB>(n_here, wsum, &total);
        const bool ok = __syncthreads_count(bad) == 0 && blk0 <= blk1 && blk1 <= d.n && total == blk1 - blk0;
        if (!ok) {
            if (tid == 0) atomicAdd(status, 1ull);
            __syncthreads();                              // wsum reused by the next block
            continue;
        }
        for (uint32_t base = 0; base < total; base += kStageSyms) {
            const uint32_t lim = total - base < (uint32_t)kStageSyms ? total - base : (uint32_t)kStageSyms;
            const uint64_t j_start = blk0 + base, j_end = j_start + lim;
            const uint32_t shift = (uint32_t)(j_start & 15);          // stage aligned to 16 elements
            // emit this round's symbols into the stage
            if (total <= (uint32_t)kStageSyms) {          // one round: every symbol has its slot
                uint32_t p = gap, k = off + shift;
                const uint32_t dummy = kStageSyms + 31;   // slot for an uncounted second codeword
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t plim = end < 32u * (q + 1) ? end : 32u * (q + 1);
                    const uint64_t pair = ((uint64_t)W[q] << 32) | W[q + 1];
                    while (p < plim) {
                        const uint32_t e = lookup(tab, tab_n, (uint32_t)((pair << (p - 32u * q)) >> 32));
                        const bool two = ((e >> 5) & 3u) == 2u && p + ((e >> 7) & 31u) < end;
                        stage[k] = (uint8_t)(e >> 12);
                        stage[two ? k + 1 : dummy] = (uint8_t)(e >> 20);
                        k += two ? 2u : 1u;
                        p += e & 31u;
                    }
                }
            } else if (off < base + lim && off + n_here > base) {
                uint32_t p = gap, k = off;                // k: output index of the next symbol
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t plim = end < 32u * (q + 1) ? end : 32u * (q + 1);
                    const uint64_t pair = ((uint64_t)W[q] << 32) | W[q + 1];
                    while (p < plim && k < base + lim) {
                        const uint32_t e = lookup(tab, tab_n, (uint32_t)((pair << (p - 32u * q)) >> 32));
                        const uint32_t nb = e & 31u, l1 = (e >> 7) & 31u;
                        if (k >= base) stage[k - base + shift] = (uint8_t)(e >> 12);
                        ++k;
                        if (((e >> 5) & 3u) == 2u && p + l1 < end) {
                            if (k >= base && k < base + lim) stage[k - base + shift] = (uint8_t)(e >> 20);
                            ++k;
                        }
                        p += nb;
                    }
                }
            }
            __syncthreads();
            // write back: whole aligned groups of 16 elements with 16-byte
            // accesses, the ragged head and tail one element per lane
            const uint64_t g_lo = (j_start + 15) >> 4, g_hi = j_end >> 4;
            const uint64_t head_end = g_lo <= g_hi ? 16 * g_lo : j_end;
            const uint64_t tail_start = g_lo <= g_hi ? 16 * g_hi : j_end;
            const uint32_t n_head = (uint32_t)(head_end - j_start), n_tail = (uint32_t)(j_end - tail_start);
            const uint64_t sbase = j_start & ~15ull;      // element at stage[0]
            if ((uint32_t)tid < n_head + n_tail) {
                const uint64_t j = (uint32_t)tid < n_head ? j_start + tid : tail_start + (tid - n_head);
                const uint32_t sy = stage[j - sbase];
                if (kFmt == ECF8V_BF16) {
                    const uint32_t r = d.raw[j];
                    reinterpret_cast<uint16_t*>(d.out)[j] = (uint16_t)(((r >> 7) << 15) | (sy << 7) | (r & 127u));
                } else {
                    const uint32_t r = (d.raw[j >> 1] >> (4 * (uint32_t)(j & 1))) & 15u;
                    d.out[j] = (uint8_t)(((r >> 2) << 7) | (sy << 2) | (r & 3u));
                }
            }
            for (uint64_t g = g_lo + tid; g < g_hi; g += kTB) {
                const uint4 sv = *reinterpret_cast<const uint4*>(stage + (16 * g - sbase));
                const uint32_t S[4] = {sv.x, sv.y, sv.z, sv.w};
                if (kFmt == ECF8V_BF16) {
                    const uint4 rv = *reinterpret_cast<const uint4*>(d.raw + 16 * g);
                    const uint32_t R[4] = {rv.x, rv.y, rv.z, rv.w};
                    uint32_t o[8];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {     // elements 4q + 2h, 4q + 2h + 1 into one word
                            const uint32_t sel = h ? 0x0c030c02u : 0x0c010c00u;
                            const uint32_t rr = __builtin_amdgcn_perm(0u, R[q], sel);
                            const uint32_t ss = __builtin_amdgcn_perm(0u, S[q], sel);
                            o[2 * q + h] = ((rr & 0x00800080u) << 8) | (ss << 7) | (rr & 0x007F007Fu);
                        }
                    }
                    uint4* dst = reinterpret_cast<uint4*>(d.out + 32 * g);
                    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
                    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
                } else {
                    const uint2 rv = *reinterpret_cast<const uint2*>(d.raw + 8 * g);
                    uint32_t o[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint32_t t = ((q < 2 ? rv.x : rv.y) >> (16 * (q & 1))) & 0xFFFFu;   // 4 nibbles
                        t = (t | (t << 8)) & 0x00FF00FFu;
                        t = (t | (t << 4)) & 0x0F0F0F0Fu;                               // one per byte
                        o[q] = ((t & 0x04040404u) << 5) | ((S[q] & 0x1F1F1F1Fu) << 2) | (t & 0x03030303u);
                    }
                    *reinterpret_cast<uint4*>(d.out + 16 * g) = make_uint4(o[0], o[1], o[2], o[3]);
                }
            }
            __syncthreads();
        }
    }
}

int check(hipError_t e) { return e == hipSuccess ? ECF8_OK : ECF8_ERR_HIP; }

template <int kFmt, int kTB>
const void* decode_kernel_ptr()
{
    return reinterpret_cast<const void*>(ecf8v_decode_kernel<kFmt, kTB>);
}

const void* pick_kernel(uint32_t fmt, uint32_t tb)
{
    if (fmt == ECF8V_BF16) {
        if (tb == 64) return decode_kernel_ptr<ECF8V_BF16, 64>();
        if (tb == 128) return decode_kernel_ptr<ECF8V_BF16, 128>();
        if (tb == 256) return decode_kernel_ptr<ECF8V_BF16, 256>();
    } else if (fmt == ECF8V_E5M2) {
        if (tb == 64) return decode_kernel_ptr<ECF8V_E5M2, 64>();
        if (tb == 128) return decode_kernel_ptr<ECF8V_E5M2, 128>();
        if (tb == 256) return decode_kernel_ptr<ECF8V_E5M2, 256>();
    }
    return nullptr;
}

std::mutex g_mu;
std::map<std::tuple<int, uint32_t, uint32_t, uint32_t>, uint32_t> g_slots;   // (device, fmt, tb, lds): workgroups

// Resident decode workgroups of the current device for a kernel and its dynamic LDS.
int kernel_slots(uint32_t fmt, uint32_t tb, uint32_t lds, uint32_t* out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ECF8_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    const auto key = std::make_tuple(dev, fmt, tb, lds);
    auto it = g_slots.find(key);
    if (it == g_slots.end()) {
        int cus = 0, occ = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return ECF8_ERR_HIP;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, pick_kernel(fmt, tb), (int)tb, lds) != hipSuccess)
            return ECF8_ERR_HIP;
        it = g_slots.emplace(key, (uint32_t)((cus > 0 ? cus : 1) * (occ > 0 ? occ : 1))).first;
    }
    *out = it->second;
    return ECF8_OK;
}

// Entries of a tensor's decode table (the layout the table kernel builds:
// 1024 primary entries plus one subtable per prefix of codewords longer than
// 10 bits, sized by the longest of them), rounded up to 4.
uint32_t table_entries(const uint8_t* len)
{
    uint32_t code[ECF8V_MAX_SYM];
    if (ecf8v_canonical_codes(len, ECF8V_MAX_SYM, code) != ECF8_OK) return 0;
    uint8_t dmax[1 << kPrimBits] = {0};
    for (int s = 0; s < ECF8V_MAX_SYM; ++s)
        if (len[s] > kPrimBits) {
            const uint32_t pre = code[s] >> (len[s] - kPrimBits);
            if (len[s] > dmax[pre]) dmax[pre] = len[s];
        }
    uint32_t used = 1u << kPrimBits;
    for (int i = 0; i < (1 << kPrimBits); ++i)
        if (dmax[i]) used += 1u << (dmax[i] - kPrimBits);
    return (used + 3) & ~3u;
}

uint32_t decode_lds_bytes(uint32_t tab_n) { return (uint32_t)(kStageSyms + 32) + 4 * tab_n; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" uint64_t ecf8v_workspace_bytes(int count)
{
    if (count < 0) return 0;
    return table_offset(count) + (uint64_t)count * kTabEntries * 4;
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
    uint32_t tab_n = 4;
    uint32_t fmt = count ? descs[0].meta.format : ECF8V_BF16, tb = count ? descs[0].meta.threads_per_block : 256;
    for (int i = 0; i < count; ++i) {
        const ecf8v_tensor_desc& t = descs[i];
        int rc = ecf8v_validate_meta(&t.meta);
        if (rc) return rc;
        if (t.meta.format != fmt || t.meta.threads_per_block != tb) return ECF8_ERR_ARG;
        if (t.meta.chunk_bytes != (uint32_t)kChunk || !pick_kernel(fmt, tb)) return ECF8_ERR_UNSUPPORTED;
        if (t.meta.n && (!t.stream || !t.raw || !t.gaps || !t.blk_off)) return ECF8_ERR_ARG;
        if (!aligned(t.stream, 16) || !aligned(t.blk_off, 8) || (t.out_offset & 15) ||
            !aligned(t.raw, fmt == ECF8V_BF16 ? 16 : 8))
            return ECF8_ERR_ARG;
        DescV& d = dv[i];
        std::memset(&d, 0, sizeof(d));
        d.stream = t.stream;
        d.raw = t.raw;
        d.gaps = t.gaps;
        d.blk_off = t.blk_off;
        d.out = out_base + t.out_offset;
        d.n = t.meta.n;
        d.n_blocks = t.meta.n ? t.meta.n_blocks : 0;
        d.first_block = blocks;
        d.total_bits = t.meta.total_bits;
        std::memcpy(d.len, t.meta.len, sizeof(d.len));
        blocks += d.n_blocks;
        if (d.n_blocks) {
            const uint32_t te = table_entries(t.meta.len);
            if (te == 0 || te > (uint32_t)kTabEntries) return ECF8_ERR_UNSUPPORTED;
            if (te > tab_n) tab_n = te;
        }
    }
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (count && hipMemcpy(ws + desc_offset(), dv.data(), sizeof(DescV) * count, hipMemcpyHostToDevice) != hipSuccess)
        return ECF8_ERR_HIP;
    // the decode tables depend on the code lengths only: built once here
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    auto* status = reinterpret_cast<unsigned long long*>(ws);
    hipLaunchKernelGGL(ecf8v_clear_kernel, dim3(1), dim3(64), 0, st, status, 2u);
    if (count)
        hipLaunchKernelGGL(ecf8v_table_kernel, dim3((uint32_t)count), dim3(256), 0, st,
                           reinterpret_cast<const DescV*>(ws + desc_offset()),
                           reinterpret_cast<uint32_t*>(ws + table_offset(count)), status);
    if (hipGetLastError() != hipSuccess || hipStreamSynchronize(st) != hipSuccess) return ECF8_ERR_HIP;
    plan->workspace = workspace;
    plan->workspace_bytes = workspace_bytes;
    plan->total_blocks = blocks;
    plan->count = (uint32_t)count;
    plan->format = fmt;
    plan->threads_per_block = tb;
    plan->table_entries = tab_n;
    uint32_t slots = 1;
    if (blocks) {
        int rc = kernel_slots(fmt, tb, decode_lds_bytes(tab_n), &slots);
        if (rc) return rc;
    }
    plan->grid = (uint32_t)(blocks < slots ? (blocks ? blocks : 1) : slots);
    return ECF8_OK;
}

extern "C" int ecf8v_decode_run(const ecf8v_plan* plan, void* hip_stream)
{
    if (!plan || !plan->workspace || plan->grid == 0) return ECF8_ERR_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    uint8_t* ws = static_cast<uint8_t*>(plan->workspace);
    auto* status = reinterpret_cast<unsigned long long*>(ws);
    const DescV* descs = reinterpret_cast<const DescV*>(ws + desc_offset());
    uint32_t* tables = reinterpret_cast<uint32_t*>(ws + table_offset((int)plan->count));
    hipLaunchKernelGGL(ecf8v_clear_kernel, dim3(1), dim3(64), 0, st, status, 1u);
    if (plan->count == 0 || plan->total_blocks == 0) return check(hipGetLastError());
    const uint32_t tb = plan->threads_per_block;
    const void* k = pick_kernel(plan->format, tb);
    if (!k) return ECF8_ERR_UNSUPPORTED;
    int count = (int)plan->count;
    uint64_t total = plan->total_blocks;
    uint32_t tab_n = plan->table_entries;
    if (tab_n < 4 || tab_n > (uint32_t)kTabEntries || (tab_n & 3)) return ECF8_ERR_ARG;
    void* args[] = {(void*)&descs, (void*)&count, (void*)&tables, (void*)&total, (void*)&status, (void*)&tab_n};
    if (hipLaunchKernel(k, dim3(plan->grid), dim3(tb), args, decode_lds_bytes(tab_n), st) != hipSuccess)
        return ECF8_ERR_HIP;
    return check(hipGetLastError());
}

extern "C" int ecf8v_decode_status(const void* workspace, void* hip_stream, uint64_t* bad_blocks)
{
    if (!workspace || !bad_blocks) return ECF8_ERR_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (hipStreamSynchronize(st) != hipSuccess) return ECF8_ERR_HIP;
    unsigned long long v[2] = {0, 0};
    if (hipMemcpy(v, workspace, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return ECF8_ERR_HIP;
    *bad_blocks = v[0] + v[1];
    return *bad_blocks ? ECF8_ERR_CORRUPT : ECF8_OK;
}
