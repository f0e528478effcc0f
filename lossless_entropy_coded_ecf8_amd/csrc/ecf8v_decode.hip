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
// Decode table (one per tensor, built on the GPU from the code lengths):
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
// again writing each symbol byte into LDS at its scanned position; the
// workgroup then assembles the output elements from the symbol and the raw
// plane and stores them.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
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
    __syncthreads();
    if (tid == 0) {
        for (int l = 0; l < 18; ++l) cnt[l] = 0;
        for (int s = 0; s < ECF8V_MAX_SYM; ++s) cnt[L[s]]++;
        cnt[0] = 0;
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
    if (tid == 0) {
        uint32_t next = 1 << kPrimBits;
        for (int i = 0; i < (1 << kPrimBits); ++i) {
            const uint32_t dm = dmax32[i];
            dmax[i] = (uint8_t)(dm ? dm - kPrimBits : 0);
            sub_base[i] = (uint16_t)(next < 65535 ? next : 65535);
            if (dm) next += 1u << (dm - kPrimBits);
        }
        used = next;
        if (next > (uint32_t)kTabEntries) atomicAdd(status + 1, 1ull);
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

__global__ __launch_bounds__(64) void ecf8v_clear_kernel(unsigned long long* status)
{
    if (threadIdx.x < 2) status[threadIdx.x] = 0ull;
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

// A lane's chunk: 20 big-endian bytes as five words, shifted out as the walk
// advances (w[0] holds the word at the current position).
struct Chunk {
    uint32_t w[5];
};

__device__ __forceinline__ uint32_t window(const Chunk& c, uint32_t o)
{
    return (uint32_t)(((((uint64_t)c.w[0] << 32) | c.w[1]) << o) >> 32);
}

__device__ __forceinline__ void advance(Chunk& c, bool adv)
{
    c.w[0] = adv ? c.w[1] : c.w[0];
    c.w[1] = adv ? c.w[2] : c.w[1];
    c.w[2] = adv ? c.w[3] : c.w[2];
    c.w[3] = adv ? c.w[4] : c.w[3];
    c.w[4] = adv ? 0u : c.w[4];
}

// Table lookup at the window; returns the symbols entry (0 = no codeword).
__device__ __forceinline__ uint32_t lookup(const uint32_t* tab, uint32_t win)
{
    uint32_t e = tab[win >> (32 - kPrimBits)];
    if (e & 0x80000000u) {
        const uint32_t k = (e >> 16) & 15u;
        e = tab[((e & 0xFFFFu) + ((win << kPrimBits) >> (32 - k))) & (kTabEntries - 1)];
        if (e & 0x80000000u) e = 0;
    }
    return (e & 31u) ? e : 0u;
}

template <int kFmt, int kTB>
__global__ __launch_bounds__(256) void ecf8v_decode_kernel(const DescV* __restrict__ descs, int count,
                                                           const uint32_t* __restrict__ tables, uint64_t total_blocks,
                                                           unsigned long long* __restrict__ status)
{
    __shared__ uint32_t tab[kTabEntries];
    __shared__ uint8_t stage[kStageSyms];
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
            for (int i = tid; i < kTabEntries / 4; i += kTB) reinterpret_cast<uint4*>(tab)[i] = src[i];
            __syncthreads();
        }
        const DescV& d = descs[t];
        const uint64_t lb = gb - t_first;
        const uint64_t blk0 = d.blk_off[lb], blk1 = d.blk_off[lb + 1];
        const uint64_t c = lb * kTB + tid;                // chunk of this lane
        const uint4 v = *reinterpret_cast<const uint4*>(d.stream + c * kChunk);
        Chunk ch0;
        ch0.w[0] = bswap(v.x);
        ch0.w[1] = bswap(v.y);
        ch0.w[2] = bswap(v.z);
        ch0.w[3] = bswap(v.w);
        ch0.w[4] = bswap(ld_u32(d.stream + (c + 1) * kChunk));
        const uint32_t gap = (d.gaps[c >> 1] >> (4 * (uint32_t)(c & 1))) & 15u;
        // codewords start before the chunk end and before T
        const uint64_t cstart = c * (uint64_t)kChunkBits;
        const uint32_t end = d.total_bits <= cstart ? 0u
                             : (d.total_bits - cstart < (uint64_t)kChunkBits ? (uint32_t)(d.total_bits - cstart)
                                                                            : (uint32_t)kChunkBits);

        // count the codewords that start inside the chunk
        Chunk ch = ch0;
        uint32_t pos = gap, n_here = 0;
        bool bad = false;
        while (pos < end) {
            const uint32_t e = lookup(tab, window(ch, pos & 31));
            if (!e) {
                bad = true;
                break;
            }
            const uint32_t nb = e & 31u, l1 = (e >> 7) & 31u, ns = (e >> 5) & 3u;
            n_here += 1u + ((ns == 2u && pos + l1 < end) ? 1u : 0u);
            const uint32_t np = pos + nb;
            advance(ch, (np >> 5) != (pos >> 5));
            pos = np;
        }
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
            // emit this round's symbols into the stage
            if (off < base + lim && off + n_here > base) {
                ch = ch0;
                pos = gap;
                uint32_t k = off;                         // output index of the next symbol
                while (pos < end && k < base + lim) {
                    const uint32_t e = lookup(tab, window(ch, pos & 31));
                    const uint32_t nb = e & 31u, l1 = (e >> 7) & 31u, ns = (e >> 5) & 3u;
                    if (k >= base) stage[k - base] = (uint8_t)(e >> 12);
                    ++k;
                    if (ns == 2u && pos + l1 < end) {
                        if (k >= base && k < base + lim) stage[k - base] = (uint8_t)(e >> 20);
                        ++k;
                    }
                    const uint32_t np = pos + nb;
                    advance(ch, (np >> 5) != (pos >> 5));
                    pos = np;
                }
            }
            __syncthreads();
            // write back: element j = blk0 + base + i
            const uint64_t j0 = blk0 + base;
            if (kFmt == ECF8V_BF16) {
                uint16_t* out = reinterpret_cast<uint16_t*>(d.out);
                for (uint32_t i = tid; i < lim; i += kTB) {
                    const uint64_t j = j0 + i;
                    const uint32_t r = d.raw[j], s = stage[i];
                    out[j] = (uint16_t)(((r >> 7) << 15) | (s << 7) | (r & 127u));
                }
            } else {
                for (uint32_t i = tid; i < lim; i += kTB) {
                    const uint64_t j = j0 + i;
                    const uint32_t r = (d.raw[j >> 1] >> (4 * (uint32_t)(j & 1))) & 15u, s = stage[i];
                    d.out[j] = (uint8_t)(((r >> 2) << 7) | (s << 2) | (r & 3u));
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
std::vector<std::vector<uint32_t>> g_slots;     // [device][kernel index]: resident workgroups

int kernel_slots(uint32_t fmt, uint32_t tb, uint32_t* out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ECF8_ERR_HIP;
    const int idx = (fmt == ECF8V_BF16 ? 0 : 3) + (tb == 64 ? 0 : tb == 128 ? 1 : 2);
    std::lock_guard<std::mutex> lk(g_mu);
    if ((int)g_slots.size() <= dev) g_slots.resize(dev + 1, std::vector<uint32_t>(6, 0u));
    if (g_slots[dev][idx] == 0) {
        int cus = 0, occ = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return ECF8_ERR_HIP;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, pick_kernel(fmt, tb), (int)tb, 0) != hipSuccess)
            return ECF8_ERR_HIP;
        g_slots[dev][idx] = (uint32_t)((cus > 0 ? cus : 1) * (occ > 0 ? occ : 1));
    }
    *out = g_slots[dev][idx];
    return ECF8_OK;
}

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
    uint32_t fmt = count ? descs[0].meta.format : ECF8V_BF16, tb = count ? descs[0].meta.threads_per_block : 256;
    for (int i = 0; i < count; ++i) {
        const ecf8v_tensor_desc& t = descs[i];
        int rc = ecf8v_validate_meta(&t.meta);
        if (rc) return rc;
        if (t.meta.format != fmt || t.meta.threads_per_block != tb) return ECF8_ERR_ARG;
        if (t.meta.chunk_bytes != (uint32_t)kChunk || !pick_kernel(fmt, tb)) return ECF8_ERR_UNSUPPORTED;
        if (t.meta.n && (!t.stream || !t.raw || !t.gaps || !t.blk_off)) return ECF8_ERR_ARG;
        if (!aligned(t.stream, 16) || !aligned(t.blk_off, 8) || (t.out_offset & 15)) return ECF8_ERR_ARG;
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
    }
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (count && hipMemcpy(ws + desc_offset(), dv.data(), sizeof(DescV) * count, hipMemcpyHostToDevice) != hipSuccess)
        return ECF8_ERR_HIP;
    plan->workspace = workspace;
    plan->workspace_bytes = workspace_bytes;
    plan->total_blocks = blocks;
    plan->count = (uint32_t)count;
    plan->format = fmt;
    plan->threads_per_block = tb;
    uint32_t slots = 1;
    if (blocks) {
        int rc = kernel_slots(fmt, tb, &slots);
        if (rc) return rc;
    }
    plan->grid = (uint32_t)(blocks < slots ? (blocks ? blocks : 1) : slots);
    (void)hip_stream;
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
    hipLaunchKernelGGL(ecf8v_clear_kernel, dim3(1), dim3(64), 0, st, status);
    if (plan->count == 0 || plan->total_blocks == 0) return check(hipGetLastError());
    hipLaunchKernelGGL(ecf8v_table_kernel, dim3(plan->count), dim3(256), 0, st, descs, tables, status);
    const uint32_t tb = plan->threads_per_block;
    const void* k = pick_kernel(plan->format, tb);
    if (!k) return ECF8_ERR_UNSUPPORTED;
    int count = (int)plan->count;
    uint64_t total = plan->total_blocks;
    void* args[] = {(void*)&descs, (void*)&count, (void*)&tables, (void*)&total, (void*)&status};
    if (hipLaunchKernel(k, dim3(plan->grid), dim3(tb), args, 0, st) != hipSuccess) return ECF8_ERR_HIP;
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
