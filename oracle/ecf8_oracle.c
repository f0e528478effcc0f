/*
 * ecf8_oracle.c -- plain, slow, obviously-correct CPU oracle for ECF8.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only tests/, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or helper with the HIP
 * library; both sides are written independently from the same format
 * description so that they can check each other.
 *
 * Sources (web pages on ECF8, cited by title and section):
 *   [ECF8 blog]  "ECF8浮点数压缩技术" (codearts.csdn.net), sections 3.1.1
 *                (dynamic Huffman coding of the 4-bit FP8 exponent: per-layer
 *                histogram, optimal prefix code, max code length <= 16),
 *                3.2.1 (parallel decode: per-thread chunk + stored gap, count,
 *                block reduction, cooperative decode, write back).
 *   [ECF8 paper] "To Compress or Not? Pushing the Frontier of Lossless GenAI
 *                Model Weights Compression with Exponent Concentration"
 *                (arXiv 2510.02676), abstract: lossless, bit-exact.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - the coded symbol is the raw 4-bit exponent field e = (b >> 3) & 15 of the
 *     E4M3 byte b; sign and mantissa form the raw nibble (s << 3) | m;
 *   - Huffman ties are broken on (weight, node id): leaves have id = symbol,
 *     internal nodes get ids 16, 17, ... in creation order;
 *   - codes are canonical: symbols sorted by (length, symbol), first code 0,
 *     next code = (previous + 1) << (length difference);
 *   - the bitstream is MSB-first: stream bit k is bit 7 - (k mod 8) of byte k/8;
 *   - element j's sign/mantissa nibble is in byte j/2, low nibble for even j;
 *   - chunk t covers stream bits [8Ct, 8C(t+1)); its gap is the offset from
 *     8Ct to the first codeword start at or after 8Ct, where the end of the
 *     stream T also counts as a start; chunks at or past T have gap 0;
 *     gaps are packed two per byte, low nibble for even t;
 *   - block b groups TB chunks; blk_off[b] is the number of codewords that
 *     start before bit 8*C*TB*b, and blk_off[n_blocks] = n.
 *
 * Every routine below walks the data one element / one bit at a time.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_NSYM 16
#define OR_MAXNODES 31

/* ---- byte fields of an FP8 E4M3 value (1 sign, 4 exponent, 3 mantissa) ---- */
static int or_sign(uint8_t b) { return (b >> 7) & 1; }
static int or_expo(uint8_t b) { return (b >> 3) & 15; }
static int or_mant(uint8_t b) { return b & 7; }

/* [ECF8 blog §3.1.1] step 1: count how often each exponent value occurs. */
void oracle_histogram(const uint8_t* x, uint64_t n, uint64_t freq[OR_NSYM])
{
    for (int s = 0; s < OR_NSYM; ++s) freq[s] = 0;
    for (uint64_t j = 0; j < n; ++j) freq[or_expo(x[j])] += 1;
}

/* [ECF8 blog §3.1.1] step 2: optimal prefix code (Huffman).  Repeatedly merge
 * the two live nodes with the smallest (weight, id); a symbol's code length is
 * the depth of its leaf.  Absent symbols get length 0; a single present
 * symbol gets length 1.  Returns the longest length. */
int oracle_huffman_lengths(const uint64_t freq[OR_NSYM], int len[OR_NSYM])
{
    uint64_t weight[OR_MAXNODES];
    int alive[OR_MAXNODES], parent[OR_MAXNODES];
    int live = 0, next_id = OR_NSYM;
    for (int i = 0; i < OR_MAXNODES; ++i) { alive[i] = 0; parent[i] = -1; weight[i] = 0; }
    for (int s = 0; s < OR_NSYM; ++s) {
        len[s] = 0;
        if (freq[s] > 0) { alive[s] = 1; weight[s] = freq[s]; live++; }
    }
    if (live == 0) return 0;
    if (live == 1) {
        for (int s = 0; s < OR_NSYM; ++s) if (alive[s]) len[s] = 1;
        return 1;
    }
    while (live > 1) {
        int pick[2];
        for (int k = 0; k < 2; ++k) {
            int best = -1;
            for (int i = 0; i < next_id; ++i) {
                if (!alive[i]) continue;
                if (best < 0 || weight[i] < weight[best] ||
                    (weight[i] == weight[best] && i < best))
                    best = i;
            }
            alive[best] = 0;
            pick[k] = best;
        }
        weight[next_id] = weight[pick[0]] + weight[pick[1]];
        parent[pick[0]] = next_id;
        parent[pick[1]] = next_id;
        alive[next_id] = 1;
        next_id++;
        live--;
    }
    int longest = 0;
    for (int s = 0; s < OR_NSYM; ++s) {
        if (freq[s] == 0) continue;
        int d = 0;
        for (int v = s; parent[v] >= 0; v = parent[v]) d++;
        len[s] = d;
        if (d > longest) longest = d;
    }
    return longest;
}

/* Canonical code assignment: symbols in (length, symbol) order; the first
 * gets code 0, each next one (previous + 1) shifted left by the growth in
 * length.  Returns 0, or -1 if a length is outside 0..16. */
int oracle_canonical_codes(const int len[OR_NSYM], uint32_t code[OR_NSYM])
{
    int order[OR_NSYM], k = 0;
    for (int s = 0; s < OR_NSYM; ++s) {
        code[s] = 0;
        if (len[s] < 0 || len[s] > 16) return -1;
        if (len[s] > 0) order[k++] = s;
    }
    /* insertion sort by (len, symbol) */
    for (int i = 1; i < k; ++i) {
        int v = order[i], j = i - 1;
        while (j >= 0 && (len[order[j]] > len[v] || (len[order[j]] == len[v] && order[j] > v))) {
            order[j + 1] = order[j];
            j--;
        }
        order[j + 1] = v;
    }
    uint32_t c = 0;
    for (int i = 0; i < k; ++i) {
        if (i > 0) c = (c + 1) << (len[order[i]] - len[order[i - 1]]);
        code[order[i]] = c;
    }
    return 0;
}

/* Total coded bits T = sum of code lengths over the elements. */
uint64_t oracle_total_bits(const uint8_t* x, uint64_t n, const int len[OR_NSYM])
{
    uint64_t t = 0;
    for (uint64_t j = 0; j < n; ++j) t += (uint64_t)len[or_expo(x[j])];
    return t;
}

/* Buffer sizes implied by the layout above. */
void oracle_sizes(uint64_t n, uint64_t total_bits, uint32_t chunk_bytes, uint32_t tb,
                  uint64_t* n_chunks, uint64_t* n_blocks, uint64_t* stream_bytes,
                  uint64_t* nibble_bytes, uint64_t* gap_bytes)
{
    uint64_t chunk_bits = 8ull * chunk_bytes;
    uint64_t nc = (total_bits + chunk_bits - 1) / chunk_bits;
    uint64_t nb = (nc + tb - 1) / tb;
    *n_chunks = nc;
    *n_blocks = nb;
    *stream_bytes = nb * tb * chunk_bytes + 16;     /* whole blocks + 16 guard bytes */
    *nibble_bytes = ((n + 15) / 16) * 8;            /* n rounded up to 16 elements */
    *gap_bytes = nb * tb / 2;
}

static void or_put_bit(uint8_t* stream, uint64_t pos, int bit)
{
    if (bit) stream[pos >> 3] |= (uint8_t)(1u << (7 - (pos & 7)));
}

static int or_get_bit(const uint8_t* stream, uint64_t pos)
{
    return (stream[pos >> 3] >> (7 - (pos & 7))) & 1;
}

/* [ECF8 blog §3.1.1 and §3.2.1] encode: bitstream of exponent codes, raw
 * sign/mantissa nibbles, per-chunk gaps and per-block output offsets.
 * All buffers must be zero-filled by the caller with the sizes from
 * oracle_sizes.  Returns T, or (uint64_t)-1 on a bad code. */
uint64_t oracle_encode(const uint8_t* x, uint64_t n, const int len[OR_NSYM],
                       uint32_t chunk_bytes, uint32_t tb,
                       uint8_t* stream, uint8_t* nibbles, uint8_t* gaps, uint64_t* blk_off)
{
    uint32_t code[OR_NSYM];
    if (oracle_canonical_codes(len, code) != 0) return (uint64_t)-1;
    for (uint64_t j = 0; j < n; ++j)
        if (len[or_expo(x[j])] == 0) return (uint64_t)-1;

    uint64_t T = oracle_total_bits(x, n, len);
    uint64_t n_chunks, n_blocks, sb, nbb, gb;
    oracle_sizes(n, T, chunk_bytes, tb, &n_chunks, &n_blocks, &sb, &nbb, &gb);
    uint64_t chunk_bits = 8ull * chunk_bytes;
    uint64_t block_bits = chunk_bits * tb;
    uint64_t total_chunks = n_blocks * tb;

    uint64_t pos = 0;            /* bit position of the next codeword start */
    uint64_t next_chunk = 0;     /* first chunk whose gap is not yet known */
    uint64_t next_block = 0;     /* first block whose offset is not yet known */
    for (uint64_t j = 0; j < n; ++j) {
        /* codeword j starts at pos: it is the first start at or after every
         * chunk / block boundary in (previous start, pos]. */
        while (next_chunk < total_chunks && next_chunk * chunk_bits <= pos) {
            uint64_t g = pos - next_chunk * chunk_bits;
            gaps[next_chunk >> 1] |= (uint8_t)((g & 15) << (4 * (next_chunk & 1)));
            next_chunk++;
        }
        while (next_block <= n_blocks && next_block * block_bits <= pos) {
            blk_off[next_block] = j;
            next_block++;
        }
        int e = or_expo(x[j]);
        for (int k = len[e] - 1; k >= 0; --k) or_put_bit(stream, pos++, (code[e] >> k) & 1);
        int nib = (or_sign(x[j]) << 3) | or_mant(x[j]);
        nibbles[j >> 1] |= (uint8_t)(nib << (4 * (j & 1)));
    }
    /* chunks after the last codeword start: the end of the stream T counts as
     * a start while the chunk begins before T; gap 0 afterwards. */
    while (next_chunk < total_chunks) {
        uint64_t s = next_chunk * chunk_bits;
        uint64_t g = (s < T) ? (T - s) : 0;
        gaps[next_chunk >> 1] |= (uint8_t)((g & 15) << (4 * (next_chunk & 1)));
        next_chunk++;
    }
    while (next_block <= n_blocks) {
        blk_off[next_block] = n;
        next_block++;
    }
    return T;
}

/* Bit-serial decode of one codeword at *pos: extend the code one bit at a
 * time until (length, code) names a symbol.  Returns the symbol or -1. */
static int or_read_symbol(const uint8_t* stream, uint64_t stream_bytes, uint64_t* pos,
                          const int len[OR_NSYM], const uint32_t code[OR_NSYM])
{
    uint32_t c = 0;
    for (int l = 1; l <= 16; ++l) {
        if ((*pos >> 3) >= stream_bytes) return -1;
        c = (c << 1) | (uint32_t)or_get_bit(stream, *pos);
        *pos += 1;
        for (int s = 0; s < OR_NSYM; ++s)
            if (len[s] == l && code[s] == c) return s;
    }
    return -1;
}

/* Decode `count` elements whose codewords start at bit `start_bit`, the first
 * being element `first_elem` (its nibble is read from the plane).  Writes
 * out[0..count).  Returns the bit position after the last codeword, or
 * (uint64_t)-1 on an invalid code. */
uint64_t oracle_decode_range(const uint8_t* stream, uint64_t stream_bytes,
                             const uint8_t* nibbles, const int len[OR_NSYM],
                             uint64_t start_bit, uint64_t first_elem, uint64_t count,
                             uint8_t* out)
{
    uint32_t code[OR_NSYM];
    if (oracle_canonical_codes(len, code) != 0) return (uint64_t)-1;
    uint64_t pos = start_bit;
    for (uint64_t i = 0; i < count; ++i) {
        int e = or_read_symbol(stream, stream_bytes, &pos, len, code);
        if (e < 0) return (uint64_t)-1;
        uint64_t j = first_elem + i;
        int nib = (nibbles[j >> 1] >> (4 * (j & 1))) & 15;
        int s = (nib >> 3) & 1, m = nib & 7;
        out[i] = (uint8_t)((s << 7) | (e << 3) | m);
    }
    return pos;
}

/* Whole-tensor decode [ECF8 blog §3.2.1, sequential form]. */
uint64_t oracle_decode(const uint8_t* stream, uint64_t stream_bytes, const uint8_t* nibbles,
                       uint64_t n, const int len[OR_NSYM], uint8_t* out)
{
    return oracle_decode_range(stream, stream_bytes, nibbles, len, 0, 0, n, out);
}

/* [ECF8 blog §3.2.1] the count step of the parallel decode, bit-serial: the
 * thread that owns chunk t starts at its stored gap (bit 8Ct + gap) and
 * decodes codewords one bit at a time; it counts every codeword that starts
 * before the end of its chunk, min(8C(t+1), T).  A chunk whose start is at or
 * past T counts nothing.  The stored gap is taken as given (it may be
 * corrupt), so this is also what a decoder that trusts it finds.  Returns the
 * count, or -1 if a codeword is invalid (possible only for an incomplete
 * code) or runs past the stream. */
int64_t oracle_chunk_count(const uint8_t* stream, uint64_t stream_bytes, uint64_t total_bits,
                           const int len[OR_NSYM], uint32_t chunk_bytes, uint64_t t, uint32_t gap)
{
    uint32_t code[OR_NSYM];
    if (oracle_canonical_codes(len, code) != 0) return -1;
    uint64_t chunk_bits = 8ull * chunk_bytes;
    uint64_t begin = chunk_bits * t;
    uint64_t end = begin + chunk_bits;
    if (end > total_bits) end = total_bits;
    uint64_t pos = begin + gap;
    int64_t count = 0;
    while (pos < end) {
        if (or_read_symbol(stream, stream_bytes, &pos, len, code) < 0) return -1;
        count++;
    }
    return count;
}

/* Re-derive gaps and block offsets from a bit walk of an existing stream and
 * compare them with the stored ones.  Returns 0 if all agree, else 1 + the
 * index of the first mismatching chunk (gaps) or -(1 + block) (offsets). */
int64_t oracle_check_layout(const uint8_t* stream, uint64_t stream_bytes, uint64_t n,
                            uint64_t total_bits, const int len[OR_NSYM],
                            uint32_t chunk_bytes, uint32_t tb,
                            const uint8_t* gaps, const uint64_t* blk_off)
{
    uint32_t code[OR_NSYM];
    if (oracle_canonical_codes(len, code) != 0) return -1000000000;
    uint64_t n_chunks, n_blocks, sb, nbb, gb;
    oracle_sizes(n, total_bits, chunk_bytes, tb, &n_chunks, &n_blocks, &sb, &nbb, &gb);
    uint64_t chunk_bits = 8ull * chunk_bytes, block_bits = chunk_bits * tb;
    uint64_t total_chunks = n_blocks * tb;
    uint64_t pos = 0, t = 0, b = 0;
    for (uint64_t j = 0; j <= n; ++j) {
        uint64_t start = (j < n) ? pos : total_bits;   /* T acts as a final start */
        while (t < total_chunks && t * chunk_bits <= start) {
            uint64_t g = start - t * chunk_bits;
            uint64_t stored = (gaps[t >> 1] >> (4 * (t & 1))) & 15;
            if (g > 15 || g != stored) return (int64_t)t + 1;
            t++;
        }
        while (b <= n_blocks && b * block_bits <= start) {
            if (blk_off[b] != ((j < n) ? j : n)) return -(int64_t)b - 1;
            b++;
        }
        if (j < n && or_read_symbol(stream, stream_bytes, &pos, len, code) < 0)
            return -1000000001;
    }
    while (t < total_chunks) {
        if (((gaps[t >> 1] >> (4 * (t & 1))) & 15) != 0) return (int64_t)t + 1;
        t++;
    }
    while (b <= n_blocks) {
        if (blk_off[b] != n) return -(int64_t)b - 1;
        b++;
    }
    return 0;
}
