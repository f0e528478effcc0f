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
//   * decode table: one LDS table of 8-byte entries indexed by the next 11
//     stream bits.  Each entry decodes greedily every whole codeword inside the
//     window (up to 8 symbols), so a lookup yields ~3.5-4.5 symbols for the
//     weight distributions of interest.  Codes longer than 11 bits (rare) live
//     in a second region indexed by the next 16 bits; one branch-free
//     max(prefix11, prefix16 - c) picks the region (canonical codes put every
//     long code at the top of the code space).  The table is built per tensor
//     on the GPU from the 16 code lengths by a small kernel and copied to LDS
//     by each persistent workgroup when its tensor changes.
//   * chunks: 16 bytes per lane, 256 lanes (4 wave64s) per block; the lane's
//     chunk plus one look-ahead dword are byte-swapped into a private LDS slot
//     (5 dwords, odd stride: bank-conflict free), and a 32-bit window at any
//     bit position is one ds_read2 + one v_alignbit.
//   * counts -> positions: wave64 inclusive scan with DPP row shifts and
//     readlane row carries, then a 4-entry cross-wave LDS prefix.
//   * decode: symbols of each lookup are OR-ed as packed nibbles into a
//     zeroed LDS staging area at the scanned nibble positions.  A lane's last
//     lookup may decode a few codewords that belong to the next lane; they are
//     the same symbols at the same positions, so OR-ing them twice is exact.
//   * write back: 16 elements per lane-step: 8 bytes of exponent nibbles from
//     LDS, 8 bytes of the sign/mantissa plane from HBM, SWAR byte assembly,
//     one 16-byte store; byte stores only at the two ragged block edges.
//   * one persistent dispatch walks all blocks of all tensors of a batch.
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
constexpr uint32_t kTableStrideEntries = 2304;                      // 18432 B per tensor table
constexpr int kChunk = 16;                                          // C
constexpr int kLanes = 256;                                         // TB
constexpr uint64_t kStatusBytes = 256;
constexpr int kTableThreads = 256;

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

// ------------------------------------------------------------ table kernel
// One workgroup per tensor.  Entry layout: .x = bits consumed | (symbols << 16),
// .y = symbols as nibbles, first symbol in the low nibble.
__global__ __launch_bounds__(kTableThreads) void ecf8_table_kernel(DevDesc* __restrict__ descs,
                                                                   uint2* __restrict__ tables)
{
    __shared__ uint32_t s_start[16];   // left-justified 16-bit first code of k-th codeword (canonical order)
    __shared__ uint32_t s_len[16];
    __shared__ uint32_t s_sym[16];
    __shared__ uint32_t s_info[4];     // k, p_long, cdelta, entries
    DevDesc* d = descs + blockIdx.x;
    if (threadIdx.x == 0) {
        uint32_t len[16];
        uint64_t lenpack = 0;
        for (int s = 0; s < 16; ++s) {
            len[s] = d->len[s];
            if (len[s]) lenpack |= (uint64_t)((len[s] - 1) & 15) << (4 * s);
        }
        int k = 0;
        for (uint32_t l = 1; l <= 16; ++l)
            for (int s = 0; s < 16; ++s)
                if (len[s] == l) {
                    s_sym[k] = s;
                    s_len[k] = l;
                    k++;
                }
        uint32_t code = 0;
        uint32_t p_long = 1u << kWin;
        bool found = false;
        for (int i = 0; i < k; ++i) {
            if (i > 0) code = (code + 1) << (s_len[i] - s_len[i - 1]);
            s_start[i] = code << (16 - s_len[i]);
            if (!found && s_len[i] > (uint32_t)kWin) {
                p_long = s_start[i] >> (16 - kWin);
                found = true;
            }
        }
        uint32_t cdelta = ((1u << (16 - kWin)) - 1) * p_long;
        uint32_t entries = 65536u - cdelta;      // <= kTableMax for every complete code
        if (entries > (uint32_t)kTableMax) entries = kTableMax;
        s_info[0] = k;
        s_info[1] = p_long;
        s_info[2] = cdelta;
        s_info[3] = entries;
        d->lenpack = lenpack;
        d->p_long = p_long;
        d->cdelta = (int32_t)cdelta;
        d->entries = entries;
    }
    __syncthreads();
    const int k = (int)s_info[0];
    const uint32_t p_long = s_info[1], cdelta = s_info[2], entries = s_info[3];
    uint2* tab = tables + (uint64_t)blockIdx.x * kTableStrideEntries;
    for (uint32_t idx = threadIdx.x; idx < entries; idx += kTableThreads) {
        uint32_t v, known;
        if (idx < p_long) {
            v = idx << (16 - kWin);
            known = kWin;
        } else {
            v = idx + cdelta;
            known = 16;
        }
        uint32_t pos = 0, ns = 0, sy = 0;
        while (k > 0 && ns < 8 && pos < known) {
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
        tab[idx] = make_uint2((pos ? pos : 1u) | (ns << 16), sy);
    }
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

// 8 exponent nibbles (e) + 8 sign/mantissa nibbles (nm), element i in nibble i,
// -> 8 FP8 bytes: byte = (s << 7) | (e << 3) | m with nm = (s << 3) | m.
__device__ __forceinline__ uint2 assemble8(uint32_t e, uint32_t nm)
{
    // even elements 0,2,4,6 -> bytes of ev; odd 1,3,5,7 -> bytes of od
    const uint32_t nev = (nm & 0x0F0F0F0Fu) | ((nm << 4) & 0xF0F0F0F0u);   // nibble copied to both halves
    const uint32_t nod = ((nm >> 4) & 0x0F0F0F0Fu) | (nm & 0xF0F0F0F0u);
    const uint32_t ev = ((e << 3) & 0x78787878u) | (nev & 0x87878787u);
    const uint32_t od = ((e >> 1) & 0x78787878u) | (nod & 0x87878787u);
    uint2 r;
    r.x = (ev & 0xFFu) | ((od & 0xFFu) << 8) | ((ev & 0xFF00u) << 8) | ((od & 0xFF00u) << 16);
    r.y = ((ev >> 16) & 0xFFu) | ((od >> 8) & 0xFF00u) | (ev & 0xFF000000u) >> 8 | (od & 0xFF000000u);
    return r;
}

// ------------------------------------------------------------ decode kernel
template <int C, int TB>
struct DecodeLds {
    static constexpr int kSlot = C / 4 + 1;                                   // dwords per lane slot
    static constexpr int kStreamDw = 1 + TB * kSlot;
    static constexpr int kOutDw = ((8 * C * TB + 15 + 8 + 16) / 8 + 2 + 3) / 4 * 4;   // nibble staging
};

template <int C, int TB>
__global__ __launch_bounds__(TB) void ecf8_decode_kernel(const DevDesc* __restrict__ descs, int count,
                                                         uint64_t total_blocks,
                                                         const uint2* __restrict__ tables,
                                                         unsigned long long* __restrict__ status)
{
    using L = DecodeLds<C, TB>;
    constexpr int kWaves = TB / 64;
    __shared__ uint2 s_table[kTableMax];
    __shared__ uint32_t s_stream[L::kStreamDw];
    __shared__ __align__(16) uint32_t s_out[L::kOutDw];
    __shared__ uint32_t s_wsum[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t* const slot_m1 = s_stream + tid * L::kSlot;   // dword before this lane's slot

    int cur = -1;
    int t = 0;
    for (uint64_t blk = blockIdx.x; blk < total_blocks; blk += gridDim.x) {
        while (t + 1 < count && blk >= descs[t].block_end) t++;
        const DevDesc* d = descs + t;
        if (t != cur) {
            __syncthreads();
            uint32_t ne = d->entries;
            if (ne == 0) {               // tables were never built for this plan: flag and skip
                if (tid == 0) atomicAdd(status, 1ull);
                continue;
            }
            ne = ne < (uint32_t)kTableMax ? ne : (uint32_t)kTableMax;
            const uint2* tab = tables + (uint64_t)t * kTableStrideEntries;
            for (uint32_t i = tid; i < ne; i += TB) s_table[i] = tab[i];
            cur = t;
            __syncthreads();
        }
        const uint64_t b = blk - d->block_begin;
        const uint64_t chunk = b * TB + tid;
        const uint64_t T = d->total_bits;
        const uint64_t cstart = chunk * (8ull * C);
        const uint32_t E = cstart >= T ? 0u : (uint32_t)((T - cstart) < 8ull * C ? (T - cstart) : 8ull * C);
        const uint32_t gap = ((uint32_t)d->gaps[chunk >> 1] >> ((chunk & 1) * 4)) & 15u;
        const uint4 sv = *reinterpret_cast<const uint4*>(d->stream + chunk * C);
        const uint32_t la = *reinterpret_cast<const uint32_t*>(d->stream + chunk * C + C);
        slot_m1[1] = __builtin_bswap32(sv.x);
        slot_m1[2] = __builtin_bswap32(sv.y);
        slot_m1[3] = __builtin_bswap32(sv.z);
        slot_m1[4] = __builtin_bswap32(sv.w);
        slot_m1[5] = __builtin_bswap32(la);
        const uint64_t lo = d->blk_off[b];
        const uint64_t hi_raw = d->blk_off[b + 1];
        const int cd = d->cdelta;
        const uint64_t lenpack = d->lenpack;

        // ---- phase 2: count the codewords that start inside [gap, E)
        const uint32_t pend = E + 31;
        uint32_t p = gap + 31;              // bit position + 31 (see window below)
        uint32_t cnt = 0, last_p = 0, last_idx = 0;
        while (p < pend) {
            // window of 32 stream bits starting at bit p - 31:
            // dwords (p >> 5) - 1 and (p >> 5) of the slot, shifted by (-(p-31)) & 31
            const uint32_t w0 = slot_m1[p >> 5];
            const uint32_t w1 = slot_m1[(p >> 5) + 1];
            const uint32_t win = __builtin_amdgcn_alignbit(w0, w1, ~p);
            const int idx = max((int)(win >> (32 - kWin)), (int)(win >> 16) - cd);
            const uint32_t ex = s_table[idx].x;
            last_p = p;
            last_idx = (uint32_t)idx;
            p += ex & 0xFFFFu;
            cnt += ex >> 16;
        }
        if (last_p) {
            // the last lookup may have decoded codewords that start at or after E
            const uint2 e = s_table[last_idx];
            const uint32_t room = pend - last_p;
            const uint32_t ns = e.x >> 16;
            uint32_t sy = e.y, start = 0, keep = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if ((uint32_t)i < ns) {
                    keep += start < room ? 1u : 0u;
                    start += (uint32_t)((lenpack >> (4 * (sy & 15))) & 15) + 1;
                    sy >>= 4;
                }
            }
            cnt -= ns - keep;
        }

        // ---- phase 3: block-wide exclusive scan of the counts
        const uint32_t incl = wave_inclusive_scan(cnt, lane);
        if (lane == 63) s_wsum[wave] = incl;
        __syncthreads();
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t s = s_wsum[w];
            before += (w < wave) ? s : 0u;
            total += s;
        }
        const uint32_t pos = before + incl - cnt;
        for (int i = tid; i < L::kOutDw / 4; i += TB) reinterpret_cast<uint4*>(s_out)[i] = make_uint4(0, 0, 0, 0);
        __syncthreads();

        // ---- phase 4: cooperative decode into the LDS staging (packed nibbles)
        const uint32_t a0 = (uint32_t)(lo & 15);
        uint32_t o = a0 + pos;
        p = gap + 31;
        while (p < pend) {
            const uint32_t w0 = slot_m1[p >> 5];
            const uint32_t w1 = slot_m1[(p >> 5) + 1];
            const uint32_t win = __builtin_amdgcn_alignbit(w0, w1, ~p);
            const int idx = max((int)(win >> (32 - kWin)), (int)(win >> 16) - cd);
            const uint2 e = s_table[idx];
            const uint64_t v = (uint64_t)e.y << ((o & 7) * 4);
            const uint32_t wa = o >> 3;
            atomicOr(&s_out[wa], (uint32_t)v);
            atomicOr(&s_out[wa + 1], (uint32_t)(v >> 32));
            o += e.x >> 16;
            p += e.x & 0xFFFFu;
        }
        __syncthreads();

        // ---- phase 5: write back [lo, hi) of this tensor
        const uint64_t n = d->n;
        const uint64_t hi = hi_raw < n ? hi_raw : n;
        const uint64_t lo_c = lo < hi ? lo : hi;
        const uint64_t want = hi - lo_c;
        if (tid == 0 && want != total) atomicAdd(status, 1ull);
        const uint32_t cap = 8u * C * TB;
        const uint32_t nw = want < cap ? (uint32_t)want : cap;
        const uint64_t base = lo_c & ~15ull;
        const uint32_t groups = ((uint32_t)(lo_c - base) + nw + 15) >> 4;
        const uint64_t end = lo_c + nw;
        const uint8_t* __restrict__ nib = d->nibbles;
        uint8_t* __restrict__ out = d->out;
        for (uint32_t g = tid; g < groups; g += TB) {
            const uint2 ex = reinterpret_cast<const uint2*>(s_out)[g];
            const uint64_t e0 = base + 16ull * g;
            const uint2 nv = *reinterpret_cast<const uint2*>(nib + (e0 >> 1));
            const uint2 r0 = assemble8(ex.x, nv.x);
            const uint2 r1 = assemble8(ex.y, nv.y);
            if (e0 >= lo_c && e0 + 16 <= end) {
                *reinterpret_cast<uint4*>(out + e0) = make_uint4(r0.x, r0.y, r1.x, r1.y);
            } else {
                const uint32_t wv[4] = {r0.x, r0.y, r1.x, r1.y};
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const uint64_t j = e0 + k;
                    if (j >= lo_c && j < end) out[j] = (uint8_t)(wv[k >> 2] >> (8 * (k & 3)));
                }
            }
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
    return table_offset(count) + (uint64_t)count * kTableStrideEntries * sizeof(uint2);
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
    uint2* tables = reinterpret_cast<uint2*>(ws + table_offset((int)plan->count));
    hipLaunchKernelGGL(ecf8_table_kernel, dim3(plan->count), dim3(kTableThreads), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), dd, tables);
    return hipGetLastError() == hipSuccess ? ECF8_OK : ECF8_ERR_HIP;
}

extern "C" int ecf8_decode_blocks(const ecf8_plan* plan, void* hip_stream)
{
    int rc = check_plan(plan);
    if (rc || plan->count == 0 || plan->total_blocks == 0) return rc;
    unsigned char* ws = static_cast<unsigned char*>(plan->workspace);
    DevDesc* dd = reinterpret_cast<DevDesc*>(ws + desc_offset());
    uint2* tables = reinterpret_cast<uint2*>(ws + table_offset((int)plan->count));
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
