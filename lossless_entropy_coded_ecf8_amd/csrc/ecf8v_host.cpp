// ecf8v_host.cpp -- host side of the BF16 (DFloat11 layout) and FP8 E5M2
// variants: exponent histogram, optimal length-limited code lengths
// (package-merge), canonical codes, sizes, metadata validation and the
// multithreaded encoder (include/ecf8v.h).
//
// Method: the DFloat11 article §2 -- per-tensor statistics of the exponent
// values, Huffman codes for the exponent, sign and mantissa kept; the ECF8
// technical blog §3.1.1 -- code lengths limited to 16 bits -- and §3.2.1 --
// the chunk / gap / block layout the decoder walks.  The length limit is met
// optimally by package-merge (Larmore and Hirschberg, J. ACM 37(3), 1990).
#include "ecf8v.h"
#include "host_threads.h"

#include <algorithm>
#include <cstring>
#include <vector>

namespace {

using ecf8_host::run_parallel;
using ecf8_host::worker_count;

constexpr int kMaxLen = 16;

bool format_ok(uint32_t f) { return f == ECF8V_BF16 || f == ECF8V_E5M2; }
int nsym_of(uint32_t f) { return f == ECF8V_BF16 ? 256 : 32; }

// Exponent symbol and raw field of element j.
inline uint32_t bf16_at(const void* d, uint64_t j) { return static_cast<const uint16_t*>(d)[j]; }
inline uint32_t e5m2_at(const void* d, uint64_t j) { return static_cast<const uint8_t*>(d)[j]; }
inline int sym_of(uint32_t f, uint32_t v) { return f == ECF8V_BF16 ? (int)((v >> 7) & 255) : (int)((v >> 2) & 31); }
inline uint32_t raw_of(uint32_t f, uint32_t v)
{
    return f == ECF8V_BF16 ? (((v >> 15) & 1u) << 7) | (v & 127u) : (((v >> 7) & 1u) << 2) | (v & 3u);
}
inline uint32_t value_at(uint32_t f, const void* d, uint64_t j) { return f == ECF8V_BF16 ? bf16_at(d, j) : e5m2_at(d, j); }

bool params_ok(const ecf8_params* p)
{
    if (!p) return false;
    if (p->chunk_bytes < 4 || p->chunk_bytes > 64 || p->chunk_bytes % 4) return false;
    if (p->threads_per_block < 64 || p->threads_per_block > 1024 || p->threads_per_block % 64) return false;
    return true;
}

// Lengths usable by the decoder: each <= 16, prefix (Kraft sum <= 1, exactly
// 1 for >= 2 present symbols, so every stream bit pattern decodes), a lone
// symbol of length 1.  Returns the longest length, or -1.
int lengths_ok(const uint8_t* len, int nsym)
{
    int present = 0, longest = 0;
    uint64_t kraft = 0;                      // in units of 2^-16
    for (int s = 0; s < nsym; ++s) {
        if (len[s] > kMaxLen) return -1;
        if (len[s]) {
            present++;
            longest = std::max<int>(longest, len[s]);
            kraft += 1ull << (kMaxLen - len[s]);
        }
    }
    if (present == 0) return 0;
    if (present == 1) return longest == 1 ? 1 : -1;
    return kraft == (1ull << kMaxLen) ? longest : -1;
}

struct Layout {
    uint64_t n_chunks, n_blocks, stream_bytes, raw_bytes, gap_bytes;
};

Layout layout_of(uint32_t f, uint64_t n, uint64_t T, uint32_t C, uint32_t TB)
{
    Layout L;
    const uint64_t chunk_bits = 8ull * C;
    L.n_chunks = (T + chunk_bits - 1) / chunk_bits;
    L.n_blocks = (L.n_chunks + TB - 1) / TB;
    L.stream_bytes = L.n_blocks * TB * C + 16;
    L.raw_bytes = ((n + 15) / 16) * (f == ECF8V_BF16 ? 16 : 8);
    L.gap_bytes = L.n_blocks * TB / 2;
    return L;
}

void histogram_mt(uint32_t f, const void* d, uint64_t n, uint64_t* freq)
{
    const int ns = nsym_of(f);
    int workers = worker_count(n, 1u << 22);
    std::vector<uint64_t> part((size_t)workers * ns, 0);
    run_parallel(workers, [&](int w) {
        uint64_t lo = n * w / workers, hi = n * (w + 1) / workers;
        uint64_t* mine = &part[(size_t)w * ns];
        if (f == ECF8V_BF16) {
            const uint16_t* x = static_cast<const uint16_t*>(d);
            for (uint64_t j = lo; j < hi; ++j) mine[(x[j] >> 7) & 255]++;
        } else {
            uint64_t local[256] = {0};
            const uint8_t* x = static_cast<const uint8_t*>(d);
            for (uint64_t j = lo; j < hi; ++j) local[x[j]]++;
            for (int b = 0; b < 256; ++b) mine[(b >> 2) & 31] += local[b];
        }
    });
    for (int s = 0; s < ns; ++s) {
        freq[s] = 0;
        for (int w = 0; w < workers; ++w) freq[s] += part[(size_t)w * ns + s];
    }
}

// Canonical codes of valid lengths: codes of each length are consecutive in
// symbol order, and each length's first code follows the previous length's
// last, shifted by the growth in length.
void canonical(const uint8_t* len, int nsym, uint32_t* code)
{
    uint32_t count[kMaxLen + 1] = {0}, next[kMaxLen + 2] = {0};
    for (int s = 0; s < nsym; ++s) count[len[s]]++;
    count[0] = 0;
    uint32_t c = 0;
    for (int l = 1; l <= kMaxLen; ++l) {
        c = (c + count[l - 1]) << 1;
        next[l] = c;
    }
    for (int s = 0; s < nsym; ++s) code[s] = len[s] ? next[len[s]]++ : 0u;
}

// Package-merge over the present symbols' weights.  Level lists run from
// max_len (the leaves alone) up to 1; each list is sorted and records, per
// item, whether it is a leaf.  The 2m - 2 cheapest items of level 1 are
// chosen; the chosen prefix of a level holds the c_d smallest leaves and p_d
// packages, which select the 2 p_d cheapest items of the level below.  A leaf
// of rank i gets length #{levels d : i < c_d}.  Ties: a leaf before a package
// of equal weight.
int package_merge(const uint64_t* freq, int nsym, int max_len, uint8_t* len)
{
    std::vector<int> sym;
    for (int s = 0; s < nsym; ++s) {
        len[s] = 0;
        if (freq[s]) sym.push_back(s);
    }
    const int m = (int)sym.size();
    if (m == 0) return ECF8_OK;
    if (m == 1) {
        len[sym[0]] = 1;
        return ECF8_OK;
    }
    if ((1ll << max_len) < m) return ECF8_ERR_UNSUPPORTED;
    std::stable_sort(sym.begin(), sym.end(), [&](int a, int b) { return freq[a] < freq[b]; });
    std::vector<uint64_t> leaf_w(m);
    for (int i = 0; i < m; ++i) leaf_w[i] = freq[sym[i]];

    std::vector<std::vector<uint8_t>> is_leaf(max_len + 1);
    std::vector<uint64_t> cur(leaf_w), nxt;
    is_leaf[max_len].assign(m, 1);
    for (int d = max_len - 1; d >= 1; --d) {
        const size_t np = cur.size() / 2;
        nxt.clear();
        is_leaf[d].clear();
        size_t a = 0, b = 0;
        while (a < (size_t)m || b < np) {
            const uint64_t pw = b < np ? cur[2 * b] + cur[2 * b + 1] : 0;
            if (b >= np || (a < (size_t)m && leaf_w[a] <= pw)) {
                nxt.push_back(leaf_w[a++]);
                is_leaf[d].push_back(1);
            } else {
                nxt.push_back(pw);
                is_leaf[d].push_back(0);
                b++;
            }
        }
        cur.swap(nxt);
    }
    std::vector<int> depth(m, 0);
    size_t take = 2 * (size_t)m - 2;
    for (int d = 1; d <= max_len && take; ++d) {
        size_t leaves = 0, packages = 0;
        for (size_t i = 0; i < take; ++i) (is_leaf[d][i] ? leaves : packages)++;
        for (size_t i = 0; i < leaves; ++i) depth[i]++;
        take = 2 * packages;
    }
    for (int i = 0; i < m; ++i) len[sym[i]] = (uint8_t)depth[i];
    return ECF8_OK;
}

// Per-segment MSB-first writer: whole bytes go straight to the stream; the
// first byte (when the segment starts mid-byte) and the last partial byte are
// kept aside because the neighbouring segments share them.
struct Edge {
    uint64_t head_at = ~0ull, tail_at = ~0ull;
    uint8_t head = 0, tail = 0;
};

}  // namespace

extern "C" int ecf8v_nsym(uint32_t format) { return format_ok(format) ? nsym_of(format) : ECF8_ERR_ARG; }

extern "C" int ecf8v_histogram(uint32_t format, const void* data, uint64_t n, uint64_t* freq)
{
    if (!format_ok(format) || !freq || (!data && n)) return ECF8_ERR_ARG;
    histogram_mt(format, data, n, freq);
    return ECF8_OK;
}

extern "C" int ecf8v_code_lengths(const uint64_t* freq, uint32_t nsym, uint32_t max_len, uint8_t* len)
{
    if (!freq || !len || nsym == 0 || nsym > ECF8V_MAX_SYM || max_len < 1 || max_len > kMaxLen) return ECF8_ERR_ARG;
    return package_merge(freq, (int)nsym, (int)max_len, len);
}

extern "C" int ecf8v_canonical_codes(const uint8_t* len, uint32_t nsym, uint32_t* code)
{
    if (!len || !code || nsym == 0 || nsym > ECF8V_MAX_SYM) return ECF8_ERR_ARG;
    uint64_t kraft = 0;
    for (uint32_t s = 0; s < nsym; ++s) {
        if (len[s] > kMaxLen) return ECF8_ERR_META;
        if (len[s]) kraft += 1ull << (kMaxLen - len[s]);
    }
    if (kraft > (1ull << kMaxLen)) return ECF8_ERR_META;
    canonical(len, (int)nsym, code);
    return ECF8_OK;
}

extern "C" int ecf8v_encode_sizes(uint32_t format, const void* data, uint64_t n, const uint8_t* len,
                                  const ecf8_params* params, ecf8v_meta* out)
{
    if (!format_ok(format) || !len || !out || (!data && n) || !params_ok(params)) return ECF8_ERR_ARG;
    const int ns = nsym_of(format);
    const int longest = lengths_ok(len, ns);
    if (longest < 0) return ECF8_ERR_META;
    std::vector<uint64_t> freq(ns);
    histogram_mt(format, data, n, freq.data());
    uint64_t T = 0;
    for (int s = 0; s < ns; ++s) {
        if (freq[s] && !len[s]) return ECF8_ERR_META;
        T += freq[s] * len[s];
    }
    Layout L = layout_of(format, n, T, params->chunk_bytes, params->threads_per_block);
    std::memset(out, 0, sizeof(*out));
    out->n = n;
    out->total_bits = T;
    out->n_chunks = L.n_chunks;
    out->n_blocks = L.n_blocks;
    out->stream_bytes = L.stream_bytes;
    out->raw_bytes = L.raw_bytes;
    out->gap_bytes = L.gap_bytes;
    out->chunk_bytes = params->chunk_bytes;
    out->threads_per_block = params->threads_per_block;
    out->format = format;
    out->max_len = n ? (uint32_t)longest : 0u;
    std::memcpy(out->len, len, (size_t)ns);
    return ECF8_OK;
}

extern "C" int ecf8v_validate_meta(const ecf8v_meta* m)
{
    if (!m) return ECF8_ERR_ARG;
    if (!format_ok(m->format)) return ECF8_ERR_META;
    ecf8_params p{m->chunk_bytes, m->threads_per_block};
    if (!params_ok(&p)) return ECF8_ERR_META;
    const int ns = nsym_of(m->format);
    for (int s = ns; s < ECF8V_MAX_SYM; ++s)
        if (m->len[s]) return ECF8_ERR_META;
    const int longest = lengths_ok(m->len, ns);
    if (longest < 0) return ECF8_ERR_META;
    if (m->n == 0) {
        if (m->total_bits || m->max_len) return ECF8_ERR_META;
    } else {
        if (longest == 0 || (uint32_t)longest != m->max_len) return ECF8_ERR_META;
        int shortest = kMaxLen;
        for (int s = 0; s < ns; ++s)
            if (m->len[s]) shortest = std::min<int>(shortest, m->len[s]);
        if (m->total_bits < m->n * (uint64_t)shortest || m->total_bits > m->n * (uint64_t)longest)
            return ECF8_ERR_META;
    }
    Layout L = layout_of(m->format, m->n, m->total_bits, m->chunk_bytes, m->threads_per_block);
    if (L.n_chunks != m->n_chunks || L.n_blocks != m->n_blocks || L.stream_bytes != m->stream_bytes ||
        L.raw_bytes != m->raw_bytes || L.gap_bytes != m->gap_bytes)
        return ECF8_ERR_META;
    return ECF8_OK;
}

extern "C" int ecf8v_encode(uint32_t format, const void* data, uint64_t n, const uint8_t* len,
                            const ecf8_params* params, uint8_t* stream, uint64_t stream_cap, uint8_t* raw,
                            uint64_t raw_cap, uint8_t* gaps, uint64_t gap_cap, uint64_t* blk_off, uint64_t blk_cap,
                            ecf8v_meta* meta)
{
    ecf8v_meta m;
    int rc = ecf8v_encode_sizes(format, data, n, len, params, &m);
    if (rc) return rc;
    if (!meta || !stream || !blk_off || (!raw && m.raw_bytes) || (!gaps && m.gap_bytes)) return ECF8_ERR_ARG;
    if (stream_cap < m.stream_bytes || raw_cap < m.raw_bytes || gap_cap < m.gap_bytes || blk_cap < m.n_blocks + 1)
        return ECF8_ERR_SIZE;
    const int ns = nsym_of(format);
    uint32_t code[ECF8V_MAX_SYM];
    canonical(len, ns, code);
    const uint64_t C = m.chunk_bytes, TB = m.threads_per_block;
    const uint64_t chunk_bits = 8 * C, block_bits = chunk_bits * TB, T = m.total_bits;
    const uint64_t total_chunks = m.n_blocks * TB;

    // segments of whole 16-element groups (the E5M2 raw plane packs two
    // elements per byte); pass 1: bits per segment
    const int workers = worker_count(n, 1u << 20);
    const int nseg = std::max(1, workers * 4);
    std::vector<uint64_t> lo(nseg + 1), bits(nseg, 0), start(nseg + 1, 0);
    const uint64_t groups = (n + 15) / 16;
    for (int i = 0; i <= nseg; ++i) lo[i] = std::min<uint64_t>(n, groups * (uint64_t)i / nseg * 16);
    run_parallel(workers, [&](int w) {
        for (int i = w; i < nseg; i += workers) {
            uint64_t b = 0;
            for (uint64_t j = lo[i]; j < lo[i + 1]; ++j) b += len[sym_of(format, value_at(format, data, j))];
            bits[i] = b;
        }
    });
    for (int i = 0; i < nseg; ++i) start[i + 1] = start[i] + bits[i];

    // pass 2: stream bits, raw plane, gaps (one byte per chunk first) and block offsets
    std::vector<uint8_t> gap1(total_chunks, 0);
    std::vector<Edge> edge(nseg);
    std::memset(raw, 0, m.raw_bytes);
    run_parallel(workers, [&](int w) {
        for (int i = w; i < nseg; i += workers) {
            const uint64_t j0 = lo[i], j1 = lo[i + 1];
            if (j0 == j1) continue;
            uint64_t p = start[i];
            // chunk and block starts at or before the previous codeword start
            // belong to earlier segments
            uint64_t t = 0, b = 0;
            if (j0 > 0) {
                const uint64_t prev = p - len[sym_of(format, value_at(format, data, j0 - 1))];
                t = prev / chunk_bits + 1;
                b = prev / block_bits + 1;
            }
            uint64_t acc = 0;                     // pending bits, left-aligned
            int nacc = (int)(p & 7);
            uint64_t at = p >> 3;
            bool head = (p & 7) != 0;
            for (uint64_t j = j0; j < j1; ++j) {
                for (; t < total_chunks && t * chunk_bits <= p; ++t) gap1[t] = (uint8_t)(p - t * chunk_bits);
                for (; b <= m.n_blocks && b * block_bits <= p; ++b) blk_off[b] = j;
                const uint32_t v = value_at(format, data, j);
                const int s = sym_of(format, v), l = len[s];
                acc |= (uint64_t)code[s] << (64 - nacc - l);
                nacc += l;
                p += l;
                for (; nacc >= 8; nacc -= 8, acc <<= 8, ++at) {
                    const uint8_t byte = (uint8_t)(acc >> 56);
                    if (head) {
                        edge[i].head_at = at;
                        edge[i].head = byte;
                        head = false;
                    } else {
                        stream[at] = byte;
                    }
                }
                const uint32_t r = raw_of(format, v);
                if (format == ECF8V_BF16)
                    raw[j] = (uint8_t)r;
                else
                    raw[j >> 1] |= (uint8_t)(r << (4 * (j & 1)));
            }
            if (nacc > 0) {
                if (head) {
                    edge[i].head_at = at;
                    edge[i].head = (uint8_t)(acc >> 56);
                } else {
                    edge[i].tail_at = at;
                    edge[i].tail = (uint8_t)(acc >> 56);
                }
            }
        }
    });
    for (const Edge& e : edge) {
        if (e.head_at != ~0ull) stream[e.head_at] = 0;
        if (e.tail_at != ~0ull) stream[e.tail_at] = 0;
    }
    for (const Edge& e : edge) {
        if (e.head_at != ~0ull) stream[e.head_at] |= e.head;
        if (e.tail_at != ~0ull) stream[e.tail_at] |= e.tail;
    }
    const uint64_t used = (T + 7) >> 3;
    std::memset(stream + used, 0, m.stream_bytes - used);
    // chunks and blocks after the last codeword start: T counts as a start
    {
        const uint64_t last = n ? T - len[sym_of(format, value_at(format, data, n - 1))] : 0;
        for (uint64_t t = n ? last / chunk_bits + 1 : 0; t < total_chunks; ++t) {
            const uint64_t s = t * chunk_bits;
            gap1[t] = (uint8_t)(s < T ? T - s : 0);
        }
        for (uint64_t b = n ? last / block_bits + 1 : 0; b <= m.n_blocks; ++b) blk_off[b] = n;
    }
    std::memset(gaps, 0, m.gap_bytes);
    for (uint64_t t = 0; t < total_chunks; t += 2)
        gaps[t >> 1] = (uint8_t)((gap1[t] & 15) | ((gap1[t + 1] & 15) << 4));
    *meta = m;
    return ECF8_OK;
}
