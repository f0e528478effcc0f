// ecf8_host.cpp -- host side of libecf8: exponent histogram, Huffman code
// lengths, canonical codes, size query, metadata validation and the
// multithreaded encoder that produces the decode-ready layout described in
// include/ecf8.h.
//
// Method: the ECF8 technical blog (codearts.csdn.net) §3.1.1 -- count the
// 4-bit exponent values of a layer, build an optimal prefix code with lengths
// limited to 16 bits, keep sign and mantissa raw; §5.1 -- the code is built
// once after training and frozen.  §3.2.1 -- the decoder gives every thread a
// chunk of the bitstream plus a stored gap (offset of its first codeword), so
// the encoder records those gaps and the per-block output offsets.
#include "ecf8.h"
#include "ecf8v.h"
#include "host_threads.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

constexpr int kNsym = ECF8_NSYM;

using ecf8_host::run_parallel;
using ecf8_host::worker_count;

inline int expo(uint8_t b) { return (b >> 3) & 15; }

// Structure of a codebook: number of present symbols, longest length, and
// whether the lengths form a prefix code that a decoder can rely on (Kraft sum
// exactly 1 for >= 2 symbols; a lone symbol has length 1).
struct CodeShape {
    int present = 0;
    int longest = 0;
    bool valid = false;
};

CodeShape shape_of(const ecf8_codebook& cb)
{
    CodeShape s;
    uint64_t kraft = 0;  // in units of 2^-16
    for (int i = 0; i < kNsym; ++i) {
        int l = cb.len[i];
        if (l == 0) continue;
        if (l > ECF8_MAX_CODE_LEN) return s;
        s.present++;
        s.longest = std::max(s.longest, l);
        kraft += 1ull << (16 - l);
    }
    if (s.present == 0) s.valid = true;
    else if (s.present == 1) s.valid = (s.longest == 1);
    else s.valid = (kraft == (1ull << 16));
    return s;
}

void canonical(const ecf8_codebook& cb, uint32_t code[kNsym])
{
    // RFC 1951 §3.2.2 construction: count codes per length, derive the first
    // code of each length, then hand out codes in symbol order per length.
    uint32_t per_len[ECF8_MAX_CODE_LEN + 1] = {0};
    for (int s = 0; s < kNsym; ++s)
        if (cb.len[s]) per_len[cb.len[s]]++;
    uint32_t next[ECF8_MAX_CODE_LEN + 2] = {0};
    uint32_t c = 0;
    for (int l = 1; l <= ECF8_MAX_CODE_LEN; ++l) {
        c = (c + per_len[l - 1]) << 1;
        next[l] = c;
    }
    for (int s = 0; s < kNsym; ++s) code[s] = cb.len[s] ? next[cb.len[s]]++ : 0;
}

struct Layout {
    uint64_t n_chunks, n_blocks, stream_bytes, nibble_bytes, gap_bytes;
};

Layout layout_of(uint64_t n, uint64_t T, uint32_t C, uint32_t TB)
{
    Layout L;
    const uint64_t chunk_bits = 8ull * C;
    L.n_chunks = T / chunk_bits + (T % chunk_bits ? 1 : 0);
    L.n_blocks = L.n_chunks / TB + (L.n_chunks % TB ? 1 : 0);
    L.stream_bytes = L.n_blocks * TB * C + 16;
    L.nibble_bytes = ((n + 15) >> 4) << 3;
    L.gap_bytes = L.n_blocks * TB / 2;
    return L;
}

bool params_ok(const ecf8_params* p)
{
    if (!p) return false;
    if (p->chunk_bytes < 4 || p->chunk_bytes > 64 || p->chunk_bytes % 4) return false;
    if (p->threads_per_block < 64 || p->threads_per_block > 1024 || p->threads_per_block % 64) return false;
    return true;
}

void histogram_mt(const uint8_t* x, uint64_t n, uint64_t freq[kNsym])
{
    int workers = worker_count(n, 1u << 22);
    std::vector<uint64_t> part((size_t)workers * kNsym, 0);
    run_parallel(workers, [&](int w) {
        uint64_t lo = n * w / workers, hi = n * (w + 1) / workers;
        uint64_t local[256] = {0};
        for (uint64_t j = lo; j < hi; ++j) local[x[j]]++;
        for (int b = 0; b < 256; ++b) part[(size_t)w * kNsym + expo((uint8_t)b)] += local[b];
    });
    for (int s = 0; s < kNsym; ++s) {
        freq[s] = 0;
        for (int w = 0; w < workers; ++w) freq[s] += part[(size_t)w * kNsym + s];
    }
}

}  // namespace

extern "C" int ecf8_alpha_hat(const float* w, uint64_t n, double gamma, double* alpha_hat)
{
    if ((!w && n) || !alpha_hat || n < 2 || !(gamma > 0.0)) return ECF8_ERR_ARG;
    double m = 0.0;
    for (uint64_t i = 0; i < n; ++i) {
        const double a = std::fabs((double)w[i]);
        if (a > m) m = a;                     // NaN compares false and is skipped
    }
    if (!(m > gamma)) return ECF8_ERR_ARG;
    *alpha_hat = std::log((double)n) / std::log(m / gamma);
    return ECF8_OK;
}

extern "C" double ecf8_exponent_entropy_bound(double alpha)
{
    if (!(alpha > 0.0)) return std::nan("");
    return alpha / (1.0 - std::exp2(-alpha));
}

extern "C" int ecf8_version(void) { return 100; }

extern "C" const char* ecf8_strerror(int code)
{
    switch (code) {
        case ECF8_OK: return "ok";
        case ECF8_ERR_ARG: return "invalid argument";
        case ECF8_ERR_SIZE: return "size mismatch";
        case ECF8_ERR_META: return "invalid metadata";
        case ECF8_ERR_UNSUPPORTED: return "unsupported parameters";
        case ECF8_ERR_CORRUPT: return "corrupt stream (decoded counts disagree with block offsets)";
        case ECF8_ERR_HIP: return "HIP runtime error";
        case ECF8_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        default: return "unknown error";
    }
}

extern "C" int ecf8_histogram(const uint8_t* fp8, uint64_t n, uint64_t freq[ECF8_NSYM])
{
    if (!freq || (!fp8 && n)) return ECF8_ERR_ARG;
    histogram_mt(fp8, n, freq);
    return ECF8_OK;
}

// Huffman lengths by the two-queue construction: leaves sorted by
// (weight, symbol), merged nodes appended in creation order (their weights
// never decrease).  Taking the smaller head by (weight, id) -- where every
// leaf id (0..15) is below every merged-node id (16..) -- selects exactly the
// node a (weight, id)-keyed priority queue would.
extern "C" int ecf8_codebook_from_freq(const uint64_t freq[ECF8_NSYM], uint32_t max_len,
                                       ecf8_codebook* out)
{
    if (!freq || !out || max_len < 1 || max_len > ECF8_MAX_CODE_LEN) return ECF8_ERR_ARG;
    std::memset(out, 0, sizeof(*out));
    int leaf_ids[kNsym], nleaf = 0;
    for (int s = 0; s < kNsym; ++s)
        if (freq[s]) leaf_ids[nleaf++] = s;
    if (nleaf == 0) return ECF8_OK;
    if (nleaf == 1) {
        out->len[leaf_ids[0]] = 1;
        return ECF8_OK;
    }
    std::sort(leaf_ids, leaf_ids + nleaf, [&](int a, int b) {
        return freq[a] != freq[b] ? freq[a] < freq[b] : a < b;
    });
    const int total = 2 * nleaf - 1;
    std::vector<uint64_t> w(16 + nleaf, 0);
    std::vector<int> parent(16 + nleaf, -1);
    for (int s = 0; s < kNsym; ++s) w[s] = freq[s];
    int lh = 0;                 // next leaf in leaf_ids
    int ih = 16, it = 16;       // merged-node queue [ih, it)
    auto take = [&]() {
        bool use_leaf;
        if (lh == nleaf) use_leaf = false;
        else if (ih == it) use_leaf = true;
        else use_leaf = w[leaf_ids[lh]] <= w[ih];   // tie -> leaf (smaller id)
        return use_leaf ? leaf_ids[lh++] : ih++;
    };
    for (int made = 0; made < nleaf - 1; ++made) {
        int a = take();
        int b = take();
        w[it] = w[a] + w[b];
        parent[a] = parent[b] = it;
        it++;
    }
    (void)total;
    int longest = 0;
    for (int s = 0; s < kNsym; ++s) {
        if (!freq[s]) continue;
        int d = 0;
        for (int v = s; parent[v] >= 0; v = parent[v]) d++;
        out->len[s] = (uint8_t)d;
        longest = std::max(longest, d);
    }
    if (longest > (int)max_len) {
        // deeper than the limit: the optimal lengths no longer than max_len
        // (package-merge, the same routine as the other float formats)
        std::memset(out, 0, sizeof(*out));
        if ((1u << max_len) < (uint32_t)nleaf) return ECF8_ERR_UNSUPPORTED;
        uint8_t len[kNsym];
        const int rc = ecf8v_code_lengths(freq, kNsym, max_len, len);
        if (rc) return rc;
        for (int s = 0; s < kNsym; ++s) out->len[s] = len[s];
    }
    return ECF8_OK;
}

extern "C" int ecf8_build_codebook(const uint8_t* fp8, uint64_t n, uint32_t max_len, ecf8_codebook* out)
{
    uint64_t freq[kNsym];
    int rc = ecf8_histogram(fp8, n, freq);
    if (rc) return rc;
    return ecf8_codebook_from_freq(freq, max_len, out);
}

extern "C" int ecf8_canonical_codes(const ecf8_codebook* cb, uint32_t code[ECF8_NSYM])
{
    if (!cb || !code) return ECF8_ERR_ARG;
    if (!shape_of(*cb).valid) return ECF8_ERR_META;
    canonical(*cb, code);
    return ECF8_OK;
}

static int sizes_from_freq(const uint64_t freq[kNsym], uint64_t n, const ecf8_codebook* cb,
                           const ecf8_params* params, ecf8_meta* out)
{
    CodeShape sh = shape_of(*cb);
    if (!sh.valid) return ECF8_ERR_META;
    uint64_t T = 0;
    for (int s = 0; s < kNsym; ++s) {
        if (freq[s] && !cb->len[s]) return ECF8_ERR_META;
        T += freq[s] * cb->len[s];
    }
    Layout L = layout_of(n, T, params->chunk_bytes, params->threads_per_block);
    std::memset(out, 0, sizeof(*out));
    out->n = n;
    out->total_bits = T;
    out->n_chunks = L.n_chunks;
    out->n_blocks = L.n_blocks;
    out->stream_bytes = L.stream_bytes;
    out->nibble_bytes = L.nibble_bytes;
    out->gap_bytes = L.gap_bytes;
    out->chunk_bytes = params->chunk_bytes;
    out->threads_per_block = params->threads_per_block;
    out->cb = *cb;
    out->max_len = (uint32_t)sh.longest;
    return ECF8_OK;
}

extern "C" int ecf8_meta_from_freq(const uint64_t freq[kNsym], uint64_t n, const ecf8_codebook* cb,
                                   const ecf8_params* params, ecf8_meta* out)
{
    if (!freq || !cb || !out || !params_ok(params)) return ECF8_ERR_ARG;
    uint64_t total = 0;
    for (int s = 0; s < kNsym; ++s) total += freq[s];
    if (total != n) return ECF8_ERR_SIZE;
    return sizes_from_freq(freq, n, cb, params, out);
}

extern "C" int ecf8_encode_sizes(const uint8_t* fp8, uint64_t n, const ecf8_codebook* cb,
                                 const ecf8_params* params, ecf8_meta* out)
{
    if (!cb || !out || (!fp8 && n) || !params_ok(params)) return ECF8_ERR_ARG;
    uint64_t freq[kNsym];
    histogram_mt(fp8, n, freq);
    return sizes_from_freq(freq, n, cb, params, out);
}

extern "C" int ecf8_validate_meta(const ecf8_meta* m)
{
    if (!m) return ECF8_ERR_ARG;
    ecf8_params p{m->chunk_bytes, m->threads_per_block};
    if (!params_ok(&p)) return ECF8_ERR_META;
    CodeShape sh = shape_of(m->cb);
    if (!sh.valid || (uint32_t)sh.longest != m->max_len) return ECF8_ERR_META;
    if (m->n == 0) {
        if (m->total_bits || m->n_chunks || m->n_blocks) return ECF8_ERR_META;
    } else {
        if (sh.present == 0) return ECF8_ERR_META;
        // every element costs between the shortest and the longest code length
        int shortest = 99;
        for (int s = 0; s < kNsym; ++s)
            if (m->cb.len[s]) shortest = std::min(shortest, (int)m->cb.len[s]);
        if (m->total_bits < m->n * (uint64_t)shortest || m->total_bits > m->n * (uint64_t)sh.longest)
            return ECF8_ERR_META;
    }
    Layout L = layout_of(m->n, m->total_bits, m->chunk_bytes, m->threads_per_block);
    if (L.n_chunks != m->n_chunks || L.n_blocks != m->n_blocks || L.stream_bytes != m->stream_bytes ||
        L.nibble_bytes != m->nibble_bytes || L.gap_bytes != m->gap_bytes)
        return ECF8_ERR_META;
    return ECF8_OK;
}

namespace {

// Per-segment MSB-first bit writer.  Whole bytes go straight to the stream;
// the first byte (if the segment starts mid-byte) and the last partial byte
// are returned separately because neighbouring segments share them.
struct SegmentOut {
    uint64_t head_index = ~0ull;
    uint8_t head = 0;
    uint64_t tail_index = ~0ull;
    uint8_t tail = 0;
};

}  // namespace

extern "C" int ecf8_encode(const uint8_t* fp8, uint64_t n, const ecf8_codebook* cb,
                           const ecf8_params* params, uint8_t* stream, uint64_t stream_cap,
                           uint8_t* nibbles, uint64_t nibble_cap, uint8_t* gaps, uint64_t gap_cap,
                           uint64_t* blk_off, uint64_t blk_cap, ecf8_meta* meta)
{
    if (!cb || !meta || (!fp8 && n) || !params_ok(params)) return ECF8_ERR_ARG;
    uint64_t freq[kNsym];
    histogram_mt(fp8, n, freq);
    ecf8_meta m;
    int rc = sizes_from_freq(freq, n, cb, params, &m);
    if (rc) return rc;
    if (!stream || !blk_off || (!nibbles && m.nibble_bytes) || (!gaps && m.gap_bytes)) return ECF8_ERR_ARG;
    if (stream_cap < m.stream_bytes || nibble_cap < m.nibble_bytes || gap_cap < m.gap_bytes ||
        blk_cap < m.n_blocks + 1)
        return ECF8_ERR_SIZE;

    const uint32_t C = params->chunk_bytes, TB = params->threads_per_block;
    const uint64_t chunk_bits = 8ull * C, block_bits = chunk_bits * TB;
    const uint64_t T = m.total_bits;
    const uint64_t total_chunks = m.n_blocks * TB;

    uint32_t code[kNsym];
    canonical(*cb, code);
    uint8_t blen[256];
    uint32_t bcode[256];
    for (int b = 0; b < 256; ++b) {
        blen[b] = cb->len[expo((uint8_t)b)];
        bcode[b] = code[expo((uint8_t)b)];
    }

    // ---- segments over elements; pass 1: bits per segment
    int workers = worker_count(n, 1u << 20);
    const int nseg = std::max(1, workers * 4);
    std::vector<uint64_t> seg_lo(nseg + 1), seg_bits(nseg + 1, 0);
    for (int i = 0; i <= nseg; ++i) seg_lo[i] = n * (uint64_t)i / nseg;
    run_parallel(workers, [&](int w) {
        for (int i = w; i < nseg; i += workers) {
            uint64_t b = 0;
            for (uint64_t j = seg_lo[i]; j < seg_lo[i + 1]; ++j) b += blen[fp8[j]];
            seg_bits[i] = b;
        }
    });
    std::vector<uint64_t> seg_start(nseg + 1, 0);
    for (int i = 0; i < nseg; ++i) seg_start[i + 1] = seg_start[i] + seg_bits[i];

    // ---- pass 2: bits, gaps (one byte per chunk first) and block offsets
    std::vector<uint8_t> gap1(total_chunks, 0);
    std::vector<SegmentOut> side(nseg);
    run_parallel(workers, [&](int w) {
        for (int i = w; i < nseg; i += workers) {
            const uint64_t j0 = seg_lo[i], j1 = seg_lo[i + 1];
            if (j0 == j1) continue;
            uint64_t p = seg_start[i];
            // boundaries already claimed by earlier segments: those at or before
            // the previous codeword start
            uint64_t t = 0, b = 0;
            if (j0 > 0) {
                uint64_t prev_start = p - blen[fp8[j0 - 1]];
                t = prev_start / chunk_bits + 1;
                b = prev_start / block_bits + 1;
            }
            uint64_t acc = 0;                 // left-aligned pending bits
            int nacc = (int)(p & 7);           // bits of the first byte owned by others
            uint64_t byte_index = p >> 3;
            bool first_byte = (p & 7) != 0;
            for (uint64_t j = j0; j < j1; ++j) {
                while (t < total_chunks && t * chunk_bits <= p) {
                    gap1[t] = (uint8_t)(p - t * chunk_bits);
                    t++;
                }
                while (b <= m.n_blocks && b * block_bits <= p) {
                    blk_off[b] = j;
                    b++;
                }
                const uint8_t x = fp8[j];
                const int l = blen[x];
                acc |= (uint64_t)bcode[x] << (64 - nacc - l);
                nacc += l;
                p += l;
                while (nacc >= 8) {
                    uint8_t byte = (uint8_t)(acc >> 56);
                    if (first_byte) {
                        side[i].head_index = byte_index;
                        side[i].head = byte;
                        first_byte = false;
                    } else {
                        stream[byte_index] = byte;
                    }
                    byte_index++;
                    acc <<= 8;
                    nacc -= 8;
                }
            }
            if (nacc > 0) {
                uint8_t byte = (uint8_t)(acc >> 56);
                if (first_byte) {  // segment never filled its first byte
                    side[i].head_index = byte_index;
                    side[i].head = byte;
                } else {
                    side[i].tail_index = byte_index;
                    side[i].tail = byte;
                }
            }
        }
    });
    // shared boundary bytes: zero them, then OR every contribution
    for (int i = 0; i < nseg; ++i) {
        if (side[i].head_index != ~0ull) stream[side[i].head_index] = 0;
        if (side[i].tail_index != ~0ull) stream[side[i].tail_index] = 0;
    }
    for (int i = 0; i < nseg; ++i) {
        if (side[i].head_index != ~0ull) stream[side[i].head_index] |= side[i].head;
        if (side[i].tail_index != ~0ull) stream[side[i].tail_index] |= side[i].tail;
    }
    const uint64_t used = (T + 7) >> 3;
    std::memset(stream + used, 0, stream_cap - used);

    // chunks after the last codeword start: T acts as a start while 8Ct < T
    {
        uint64_t last_start = n ? T - blen[fp8[n - 1]] : 0;
        uint64_t t = n ? last_start / chunk_bits + 1 : 0;
        for (; t < total_chunks; ++t) {
            uint64_t s = t * chunk_bits;
            gap1[t] = (uint8_t)(s < T ? T - s : 0);
        }
        uint64_t b = n ? last_start / block_bits + 1 : 0;
        for (; b <= m.n_blocks; ++b) blk_off[b] = n;
    }
    // pack gaps two per byte, low nibble first
    std::memset(gaps, 0, gap_cap);
    for (uint64_t t = 0; t < total_chunks; t += 2)
        gaps[t >> 1] = (uint8_t)((gap1[t] & 15) | ((gap1[t + 1] & 15) << 4));

    // ---- nibble plane: (sign << 3) | mantissa, two per byte, low nibble first
    const uint64_t pairs = n >> 1;
    run_parallel(worker_count(pairs, 1u << 22), [&](int w) {
        int ws = worker_count(pairs, 1u << 22);
        uint64_t lo = pairs * w / ws, hi = pairs * (w + 1) / ws;
        for (uint64_t k = lo; k < hi; ++k) {
            uint8_t a = fp8[2 * k], b = fp8[2 * k + 1];
            uint8_t na = (uint8_t)(((a >> 4) & 8) | (a & 7));
            uint8_t nb = (uint8_t)(((b >> 4) & 8) | (b & 7));
            nibbles[k] = (uint8_t)(na | (nb << 4));
        }
    });
    std::memset(nibbles + pairs, 0, nibble_cap - pairs);
    if (n & 1) {
        uint8_t a = fp8[n - 1];
        nibbles[pairs] = (uint8_t)(((a >> 4) & 8) | (a & 7));
    }
    *meta = m;
    return ECF8_OK;
}
