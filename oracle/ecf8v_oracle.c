/*
 * ecf8v_oracle.c -- plain, slow, obviously-correct CPU oracle for the
 * exponent-coding variants of other float formats: BF16 (the DFloat11
 * layout: 8-bit exponent coded, sign and 7 mantissa bits raw) and FP8 E5M2
 * (5-bit exponent coded, sign and 2 mantissa bits raw).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only tests/, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Sources (web pages, cited by title and section):
 *   [DF11 blog]  the DFloat11 article (BFloat16 weights), §2: per-tensor
 *                statistics of the exponent values, Huffman codes for the
 *                exponent (short codes for frequent values), sign and
 *                mantissa kept unchanged; §3.2: exponents decoded
 *                cooperatively per block, then the floats reassembled.
 *   [ECF8 blog]  "ECF8浮点数压缩技术" (codearts.csdn.net), §3.1.1: code
 *                length limited to 16 bits; §3.2.1: the chunk / gap / block
 *                layout of the stream (the same as the E4M3 oracle's).
 *   Length limiting: the pages give the limit, not the method; the optimal
 *   length-limited prefix code is computed by the package-merge algorithm
 *   (L. L. Larmore, D. S. Hirschberg, "A fast algorithm for optimal
 *   length-limited Huffman codes", J. ACM 37(3), 1990), written out here in
 *   its plainest form.
 *
 * Readings (each listed in the design notes):
 *   - BF16 value v (16 bits): symbol = (v >> 7) & 255, raw byte =
 *     (sign << 7) | (v & 127); the raw plane holds one byte per element,
 *     n rounded up to 16 elements.  (The DF11 article's struct, with an
 *     "11-bit mantissa", does not fit BF16's 7 stored mantissa bits; the
 *     plainest reading is 8 raw bits plus a coded exponent, about 11 bits.)
 *   - E5M2 byte b: symbol = (b >> 2) & 31, raw nibble = (sign << 2) | (b & 3)
 *     in the E4M3 nibble layout (element j in byte j / 2, low nibble for even
 *     j), n rounded up to 16 elements.
 *   - Huffman ties on (weight, node id), leaves having id = symbol; canonical
 *     codes in (length, symbol) order; MSB-first stream; chunk gaps, block
 *     offsets and sizes exactly as in the E4M3 oracle.
 *   - Package-merge ties: within a level, items of equal weight keep leaves
 *     (in symbol order) before packages, packages in creation order.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OV_MAXSYM 256
#define OV_MAXLEN 16

enum { OV_BF16 = 1, OV_E5M2 = 2 };

/* ---- element fields ---- */
static int ov_nsym(int fmt) { return fmt == OV_BF16 ? 256 : 32; }
static int ov_elem_bytes(int fmt) { return fmt == OV_BF16 ? 2 : 1; }

static uint32_t ov_value(int fmt, const uint8_t* x, uint64_t j)
{
    if (fmt == OV_BF16) return (uint32_t)x[2 * j] | ((uint32_t)x[2 * j + 1] << 8);   /* little-endian */
    return x[j];
}

static int ov_symbol(int fmt, uint32_t v)
{
    if (fmt == OV_BF16) return (int)((v >> 7) & 255);
    return (int)((v >> 2) & 31);
}

static uint32_t ov_raw(int fmt, uint32_t v)
{
    if (fmt == OV_BF16) return (((v >> 15) & 1) << 7) | (v & 127);
    return (((v >> 7) & 1) << 2) | (v & 3);
}

static uint32_t ov_join(int fmt, int sym, uint32_t raw)
{
    if (fmt == OV_BF16) return (((raw >> 7) & 1) << 15) | ((uint32_t)sym << 7) | (raw & 127);
    return (((raw >> 2) & 1) << 7) | ((uint32_t)sym << 2) | (raw & 3);
}

int oraclev_nsym(int fmt) { return ov_nsym(fmt); }

/* [DF11 blog §2] step 1: count how often each exponent value occurs. */
void oraclev_histogram(int fmt, const uint8_t* x, uint64_t n, uint64_t* freq)
{
    for (int s = 0; s < ov_nsym(fmt); ++s) freq[s] = 0;
    for (uint64_t j = 0; j < n; ++j) freq[ov_symbol(fmt, ov_value(fmt, x, j))] += 1;
}

/* [DF11 blog §2] step 2: Huffman code lengths, no limit.  Repeatedly merge
 * the two live nodes with the smallest (weight, id); leaves have id =
 * symbol, internal nodes nsym, nsym + 1, ... in creation order.  Absent
 * symbols get 0, a single present symbol 1.  Returns the longest length. */
int oraclev_huffman_lengths(const uint64_t* freq, int nsym, int* len)
{
    int nodes = 2 * nsym;
    uint64_t* weight = (uint64_t*)calloc((size_t)nodes, sizeof(uint64_t));
    int* alive = (int*)calloc((size_t)nodes, sizeof(int));
    int* parent = (int*)malloc((size_t)nodes * sizeof(int));
    int live = 0, next_id = nsym;
    for (int i = 0; i < nodes; ++i) parent[i] = -1;
    for (int s = 0; s < nsym; ++s) {
        len[s] = 0;
        if (freq[s] > 0) { alive[s] = 1; weight[s] = freq[s]; live++; }
    }
    int longest = 0;
    if (live == 1) {
        for (int s = 0; s < nsym; ++s) if (alive[s]) len[s] = 1;
        longest = 1;
    }
    while (live > 1) {
        int pick[2];
        for (int k = 0; k < 2; ++k) {
            int best = -1;
            for (int i = 0; i < next_id; ++i) {
                if (!alive[i]) continue;
                if (best < 0 || weight[i] < weight[best] || (weight[i] == weight[best] && i < best)) best = i;
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
    if (next_id > nsym) {
        for (int s = 0; s < nsym; ++s) {
            if (freq[s] == 0) continue;
            int d = 0;
            for (int v = s; parent[v] >= 0; v = parent[v]) d++;
            len[s] = d;
            if (d > longest) longest = d;
        }
    }
    free(weight);
    free(alive);
    free(parent);
    return longest;
}

/* One package-merge item: its weight and how many times each symbol's leaf
 * occurs inside it (a leaf is one symbol once; a package is the sum of the
 * two items it pairs). */
typedef struct {
    uint64_t weight;
    int is_leaf;
    int order;                 /* leaf: its rank in symbol order; package: creation rank */
    uint16_t count[OV_MAXSYM];
} ov_item;

static int ov_item_less(const ov_item* a, const ov_item* b)
{
    if (a->weight != b->weight) return a->weight < b->weight;
    if (a->is_leaf != b->is_leaf) return a->is_leaf;          /* leaves first on equal weight */
    return a->order < b->order;
}

/* Length-limited optimal code lengths by package-merge [ECF8 blog §3.1.1
 * limit; Larmore & Hirschberg 1990].  The "coin collector" form: the
 * present symbols' leaves are the coins of every level 1..max_len; going
 * from level max_len up to level 1, the items of the level below are paired
 * in sorted order into packages and merged with the leaves; the 2m - 2
 * cheapest items of level 1 are chosen (m present symbols); a symbol's code
 * length is how many times its leaf occurs in the chosen items.  Absent
 * symbols get 0, a single present symbol 1.  Returns the longest length, or
 * -1 if 2^max_len < m or max_len is outside 1..16. */
int oraclev_package_merge(const uint64_t* freq, int nsym, int max_len, int* len)
{
    int m = 0;
    for (int s = 0; s < nsym; ++s) {
        len[s] = 0;
        if (freq[s] > 0) m++;
    }
    if (max_len < 1 || max_len > OV_MAXLEN) return -1;
    if (m == 0) return 0;
    if (m == 1) {
        for (int s = 0; s < nsym; ++s) if (freq[s] > 0) len[s] = 1;
        return 1;
    }
    if (max_len < 31 && ((uint64_t)1 << max_len) < (uint64_t)m) return -1;

    /* the leaves, sorted by (weight, symbol) */
    ov_item* leaves = (ov_item*)calloc((size_t)m, sizeof(ov_item));
    int k = 0;
    for (int s = 0; s < nsym; ++s) {
        if (freq[s] == 0) continue;
        leaves[k].weight = freq[s];
        leaves[k].is_leaf = 1;
        leaves[k].order = s;
        leaves[k].count[s] = 1;
        k++;
    }
    for (int i = 1; i < m; ++i) {            /* insertion sort */
        ov_item v = leaves[i];
        int j = i - 1;
        while (j >= 0 && ov_item_less(&v, &leaves[j])) {
            leaves[j + 1] = leaves[j];
            j--;
        }
        leaves[j + 1] = v;
    }

    /* level max_len: the leaves alone */
    int cap = 2 * m;
    ov_item* cur = (ov_item*)calloc((size_t)cap, sizeof(ov_item));
    ov_item* nxt = (ov_item*)calloc((size_t)cap, sizeof(ov_item));
    ov_item* pk = (ov_item*)calloc((size_t)cap, sizeof(ov_item));
    int ncur = m;
    memcpy(cur, leaves, (size_t)m * sizeof(ov_item));
    for (int level = max_len - 1; level >= 1; --level) {
        /* package the items of the level below in pairs (an odd last one is dropped) */
        int np = ncur / 2;
        for (int p = 0; p < np; ++p) {
            pk[p].weight = cur[2 * p].weight + cur[2 * p + 1].weight;
            pk[p].is_leaf = 0;
            pk[p].order = p;
            for (int s = 0; s < nsym; ++s) pk[p].count[s] = (uint16_t)(cur[2 * p].count[s] + cur[2 * p + 1].count[s]);
        }
        /* merge with the leaves (both lists already sorted) */
        int a = 0, b = 0, o = 0;
        while (a < m || b < np) {
            if (b >= np || (a < m && ov_item_less(&leaves[a], &pk[b])))
                nxt[o++] = leaves[a++];
            else
                nxt[o++] = pk[b++];
        }
        ov_item* t = cur;
        cur = nxt;
        nxt = t;
        ncur = o;
    }
    /* choose the 2m - 2 cheapest items of level 1 */
    int longest = 0;
    for (int i = 0; i < 2 * m - 2; ++i)
        for (int s = 0; s < nsym; ++s) len[s] += cur[i].count[s];
    for (int s = 0; s < nsym; ++s) if (len[s] > longest) longest = len[s];
    free(leaves);
    free(cur);
    free(nxt);
    free(pk);
    return longest;
}

/* Canonical codes in (length, symbol) order; returns 0, or -1 on a length
 * outside 0..16 or an over-full code (Kraft sum > 1). */
int oraclev_canonical_codes(const int* len, int nsym, uint32_t* code)
{
    int order[OV_MAXSYM], k = 0;
    for (int s = 0; s < nsym; ++s) {
        code[s] = 0;
        if (len[s] < 0 || len[s] > OV_MAXLEN) return -1;
        if (len[s] > 0) order[k++] = s;
    }
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
        if (c >> len[order[i]]) return -1;     /* the code ran out of room */
        code[order[i]] = c;
    }
    return 0;
}

uint64_t oraclev_total_bits(int fmt, const uint8_t* x, uint64_t n, const int* len)
{
    uint64_t t = 0;
    for (uint64_t j = 0; j < n; ++j) t += (uint64_t)len[ov_symbol(fmt, ov_value(fmt, x, j))];
    return t;
}

uint64_t oraclev_raw_bytes(int fmt, uint64_t n)
{
    uint64_t groups = (n + 15) / 16;
    return fmt == OV_BF16 ? groups * 16 : groups * 8;
}

void oraclev_sizes(uint64_t total_bits, uint32_t chunk_bytes, uint32_t tb, uint64_t* n_chunks,
                   uint64_t* n_blocks, uint64_t* stream_bytes, uint64_t* gap_bytes)
{
    uint64_t chunk_bits = 8ull * chunk_bytes;
    uint64_t nc = (total_bits + chunk_bits - 1) / chunk_bits;
    uint64_t nb = (nc + tb - 1) / tb;
    *n_chunks = nc;
    *n_blocks = nb;
    *stream_bytes = nb * tb * chunk_bytes + 16;
    *gap_bytes = nb * tb / 2;
}

static void ov_put_bit(uint8_t* stream, uint64_t pos, int bit)
{
    if (bit) stream[pos >> 3] |= (uint8_t)(1u << (7 - (pos & 7)));
}

static int ov_get_bit(const uint8_t* stream, uint64_t pos) { return (stream[pos >> 3] >> (7 - (pos & 7))) & 1; }

static void ov_put_raw(int fmt, uint8_t* raw, uint64_t j, uint32_t r)
{
    if (fmt == OV_BF16)
        raw[j] = (uint8_t)r;
    else
        raw[j >> 1] |= (uint8_t)(r << (4 * (j & 1)));
}

static uint32_t ov_get_raw(int fmt, const uint8_t* raw, uint64_t j)
{
    if (fmt == OV_BF16) return raw[j];
    return (raw[j >> 1] >> (4 * (j & 1))) & 15;
}

/* Encode: exponent codes into the stream, raw fields into the raw plane,
 * per-chunk gaps and per-block offsets (the E4M3 oracle's walk).  Buffers
 * zero-filled by the caller, sized by oraclev_sizes / oraclev_raw_bytes.
 * Returns T, or (uint64_t)-1 on a bad code. */
uint64_t oraclev_encode(int fmt, const uint8_t* x, uint64_t n, const int* len, uint32_t chunk_bytes, uint32_t tb,
                        uint8_t* stream, uint8_t* raw, uint8_t* gaps, uint64_t* blk_off)
{
    int nsym = ov_nsym(fmt);
    uint32_t code[OV_MAXSYM];
    if (oraclev_canonical_codes(len, nsym, code) != 0) return (uint64_t)-1;
    for (uint64_t j = 0; j < n; ++j)
        if (len[ov_symbol(fmt, ov_value(fmt, x, j))] == 0) return (uint64_t)-1;
    uint64_t T = oraclev_total_bits(fmt, x, n, len);
    uint64_t n_chunks, n_blocks, sb, gb;
    oraclev_sizes(T, chunk_bytes, tb, &n_chunks, &n_blocks, &sb, &gb);
    uint64_t chunk_bits = 8ull * chunk_bytes, block_bits = chunk_bits * tb, total_chunks = n_blocks * tb;
    uint64_t pos = 0, next_chunk = 0, next_block = 0;
    for (uint64_t j = 0; j < n; ++j) {
        while (next_chunk < total_chunks && next_chunk * chunk_bits <= pos) {
            uint64_t g = pos - next_chunk * chunk_bits;
            gaps[next_chunk >> 1] |= (uint8_t)((g & 15) << (4 * (next_chunk & 1)));
            next_chunk++;
        }
        while (next_block <= n_blocks && next_block * block_bits <= pos) {
            blk_off[next_block] = j;
            next_block++;
        }
        uint32_t v = ov_value(fmt, x, j);
        int e = ov_symbol(fmt, v);
        for (int k = len[e] - 1; k >= 0; --k) ov_put_bit(stream, pos++, (code[e] >> k) & 1);
        ov_put_raw(fmt, raw, j, ov_raw(fmt, v));
    }
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

static int ov_read_symbol(const uint8_t* stream, uint64_t stream_bytes, uint64_t* pos, const int* len,
                          const uint32_t* code, int nsym)
{
    uint32_t c = 0;
    for (int l = 1; l <= OV_MAXLEN; ++l) {
        if ((*pos >> 3) >= stream_bytes) return -1;
        c = (c << 1) | (uint32_t)ov_get_bit(stream, *pos);
        *pos += 1;
        for (int s = 0; s < nsym; ++s)
            if (len[s] == l && code[s] == c) return s;
    }
    return -1;
}

/* Decode `count` elements from codeword bit `start_bit`, the first being
 * element `first_elem`; writes count elements of the format's size to out.
 * Returns the bit position after the last codeword, or (uint64_t)-1. */
uint64_t oraclev_decode_range(int fmt, const uint8_t* stream, uint64_t stream_bytes, const uint8_t* raw,
                              const int* len, uint64_t start_bit, uint64_t first_elem, uint64_t count, uint8_t* out)
{
    int nsym = ov_nsym(fmt);
    uint32_t code[OV_MAXSYM];
    if (oraclev_canonical_codes(len, nsym, code) != 0) return (uint64_t)-1;
    uint64_t pos = start_bit;
    for (uint64_t i = 0; i < count; ++i) {
        int e = ov_read_symbol(stream, stream_bytes, &pos, len, code, nsym);
        if (e < 0) return (uint64_t)-1;
        uint32_t v = ov_join(fmt, e, ov_get_raw(fmt, raw, first_elem + i));
        if (ov_elem_bytes(fmt) == 2) {
            out[2 * i] = (uint8_t)(v & 255);
            out[2 * i + 1] = (uint8_t)(v >> 8);
        } else {
            out[i] = (uint8_t)v;
        }
    }
    return pos;
}

uint64_t oraclev_decode(int fmt, const uint8_t* stream, uint64_t stream_bytes, const uint8_t* raw, uint64_t n,
                        const int* len, uint8_t* out)
{
    return oraclev_decode_range(fmt, stream, stream_bytes, raw, len, 0, 0, n, out);
}
