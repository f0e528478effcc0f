// exercise.cpp -- drives the host side of libecf8 (ecf8_host.cpp, ecf8v_host.cpp)
// and the CPU oracle (oracle/*.c) through a seeded set of inputs, for a build
// with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py
// compiles and runs it).  Every buffer is allocated at exactly the size the
// size query reports, so any read or write past it is caught.  The checks:
// the library's encoded bytes equal the oracle's, the oracle decodes them back
// to the input, the oracle's layout walk accepts them, and undersized buffers
// and corrupt metadata are rejected.  Exit status 0 if all pass.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ecf8.h"
#include "ecf8v.h"

extern "C" {
int oracle_huffman_lengths(const uint64_t* freq, int* len);
void oracle_histogram(const uint8_t* x, uint64_t n, uint64_t* freq);
uint64_t oracle_total_bits(const uint8_t* x, uint64_t n, const int* len);
void oracle_sizes(uint64_t n, uint64_t total_bits, uint32_t chunk_bytes, uint32_t tb, uint64_t* n_chunks,
                  uint64_t* n_blocks, uint64_t* stream_bytes, uint64_t* nibble_bytes, uint64_t* gap_bytes);
uint64_t oracle_encode(const uint8_t* x, uint64_t n, const int* len, uint32_t chunk_bytes, uint32_t tb,
                       uint8_t* stream, uint8_t* nibbles, uint8_t* gaps, uint64_t* blk_off);
uint64_t oracle_decode(const uint8_t* stream, uint64_t stream_bytes, const uint8_t* nibbles, uint64_t n,
                       const int* len, uint8_t* out);
int64_t oracle_check_layout(const uint8_t* stream, uint64_t stream_bytes, uint64_t n, uint64_t total_bits,
                            const int* len, uint32_t chunk_bytes, uint32_t tb, const uint8_t* gaps,
                            const uint64_t* blk_off);
int64_t oracle_chunk_count(const uint8_t* stream, uint64_t stream_bytes, uint64_t total_bits, const int* len,
                           uint32_t chunk_bytes, uint64_t t, uint32_t gap);
int oraclev_nsym(int fmt);
uint64_t oraclev_total_bits(int fmt, const uint8_t* x, uint64_t n, const int* len);
uint64_t oraclev_raw_bytes(int fmt, uint64_t n);
void oraclev_sizes(uint64_t total_bits, uint32_t chunk_bytes, uint32_t tb, uint64_t* n_chunks, uint64_t* n_blocks,
                   uint64_t* stream_bytes, uint64_t* gap_bytes);
uint64_t oraclev_encode(int fmt, const uint8_t* x, uint64_t n, const int* len, uint32_t chunk_bytes, uint32_t tb,
                        uint8_t* stream, uint8_t* raw, uint8_t* gaps, uint64_t* blk_off);
uint64_t oraclev_decode(int fmt, const uint8_t* stream, uint64_t stream_bytes, const uint8_t* raw, uint64_t n,
                        const int* len, uint8_t* out);
}

static int g_fail = 0;
#define CHECK(c, ...)                                                  \
    do {                                                               \
        if (!(c)) {                                                    \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);  \
            std::fprintf(stderr, __VA_ARGS__);                         \
            std::fprintf(stderr, "\n");                                \
            g_fail++;                                                  \
        }                                                              \
    } while (0)

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next64()   // splitmix64
{
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// FP8 bytes of a kind: 0 uniform bytes, 1 geometric exponents (heavy skew), 2 one exponent value
static std::vector<uint8_t> make_bytes(uint64_t n, int kind)
{
    std::vector<uint8_t> x(n);
    for (uint64_t j = 0; j < n; ++j) {
        uint64_t r = next64();
        if (kind == 0) {
            x[j] = (uint8_t)r;
        } else if (kind == 1) {
            int e = 0;
            while (e < 15 && (r & 1)) { e++; r >>= 1; }
            x[j] = (uint8_t)(((r >> 8) & 0x80) | (e << 3) | ((r >> 16) & 7));
        } else {
            x[j] = (uint8_t)(0x38 | ((r >> 8) & 0x87));
        }
    }
    return x;
}

static void e4m3_case(const std::vector<uint8_t>& x, uint32_t C, uint32_t TB)
{
    const uint64_t n = x.size();
    const uint8_t* xp = n ? x.data() : nullptr;
    ecf8_codebook cb;
    CHECK(ecf8_build_codebook(xp, n, 16, &cb) == ECF8_OK, "build_codebook n=%llu", (unsigned long long)n);
    uint64_t freq[16];
    oracle_histogram(xp, n, freq);
    int olen[16];
    oracle_huffman_lengths(freq, olen);
    for (int s = 0; s < 16; ++s) CHECK((int)cb.len[s] == olen[s], "length of symbol %d", s);
    ecf8_params p{C, TB};
    ecf8_meta m;
    CHECK(ecf8_encode_sizes(xp, n, &cb, &p, &m) == ECF8_OK, "encode_sizes");
    // exact-size buffers (at least one byte so that the pointers are valid)
    std::vector<uint8_t> stream(m.stream_bytes ? m.stream_bytes : 1), nib(m.nibble_bytes ? m.nibble_bytes : 1),
        gaps(m.gap_bytes ? m.gap_bytes : 1);
    std::vector<uint64_t> blk(m.n_blocks + 1);
    ecf8_meta m2;
    CHECK(ecf8_encode(xp, n, &cb, &p, stream.data(), m.stream_bytes, nib.data(), m.nibble_bytes, gaps.data(),
                      m.gap_bytes, blk.data(), m.n_blocks + 1, &m2) == ECF8_OK, "encode n=%llu", (unsigned long long)n);
    CHECK(ecf8_validate_meta(&m2) == ECF8_OK, "validate_meta");
    // capacities one short are rejected
    if (m.stream_bytes)
        CHECK(ecf8_encode(xp, n, &cb, &p, stream.data(), m.stream_bytes - 1, nib.data(), m.nibble_bytes, gaps.data(),
                          m.gap_bytes, blk.data(), m.n_blocks + 1, &m2) == ECF8_ERR_SIZE, "short stream");
    CHECK(ecf8_encode(xp, n, &cb, &p, stream.data(), m.stream_bytes, nib.data(), m.nibble_bytes, gaps.data(),
                      m.gap_bytes, blk.data(), m.n_blocks, &m2) == ECF8_ERR_SIZE, "short blk_off");
    // the oracle's encoding of the same bytes is identical
    uint64_t nc, nb, sb, nbb, gb;
    const uint64_t T = oracle_total_bits(xp, n, olen);
    oracle_sizes(n, T, C, TB, &nc, &nb, &sb, &nbb, &gb);
    CHECK(T == m.total_bits && nc == m.n_chunks && nb == m.n_blocks && sb == m.stream_bytes &&
          nbb == m.nibble_bytes && gb == m.gap_bytes, "sizes");
    std::vector<uint8_t> os(sb ? sb : 1, 0), on(nbb ? nbb : 1, 0), og(gb ? gb : 1, 0);
    std::vector<uint64_t> ob(nb + 1, 0);
    CHECK(oracle_encode(xp, n, olen, C, TB, os.data(), on.data(), og.data(), ob.data()) == T, "oracle_encode");
    CHECK(std::memcmp(os.data(), stream.data(), sb) == 0, "stream bytes");
    CHECK(std::memcmp(on.data(), nib.data(), nbb) == 0, "nibble bytes");
    CHECK(std::memcmp(og.data(), gaps.data(), gb) == 0, "gap bytes");
    CHECK(std::memcmp(ob.data(), blk.data(), 8 * (nb + 1)) == 0, "block offsets");
    CHECK(oracle_check_layout(stream.data(), sb, n, T, olen, C, TB, gaps.data(), blk.data()) == 0, "layout");
    std::vector<uint8_t> out(n ? n : 1);
    CHECK(oracle_decode(stream.data(), sb, nib.data(), n, olen, out.data()) != (uint64_t)-1, "oracle_decode");
    CHECK(n == 0 || std::memcmp(out.data(), x.data(), n) == 0, "round trip");
    // per-block counts from the stored gaps equal the block offsets
    for (uint64_t b = 0; b < nb; ++b) {
        int64_t tot = 0;
        for (uint64_t t = b * TB; t < (b + 1) * TB; ++t)
            tot += oracle_chunk_count(stream.data(), sb, T, olen, C, t, (gaps[t >> 1] >> (4 * (t & 1))) & 15);
        CHECK(tot == (int64_t)(blk[b + 1] - blk[b]), "block %llu count", (unsigned long long)b);
    }
    // corrupt metadata is rejected
    ecf8_meta bad = m2;
    bad.stream_bytes += 1;
    CHECK(ecf8_validate_meta(&bad) == ECF8_ERR_META, "meta stream_bytes");
    bad = m2;
    bad.cb.len[0] = 17;
    CHECK(ecf8_validate_meta(&bad) == ECF8_ERR_META, "meta length 17");
    bad = m2;
    bad.chunk_bytes = 6;
    CHECK(ecf8_validate_meta(&bad) == ECF8_ERR_META, "meta chunk 6");
}

static void variant_case(int fmt, uint64_t n, uint32_t C, uint32_t TB)
{
    const int eb = fmt == ECF8V_BF16 ? 2 : 1;
    std::vector<uint8_t> x(n * eb + 1);
    for (uint64_t j = 0; j < n; ++j) {
        uint64_t r = next64();
        int e = 0;
        while (e < (fmt == ECF8V_BF16 ? 40 : 20) && (r & 1)) { e++; r >>= 1; }
        if (fmt == ECF8V_BF16) {
            uint32_t v = ((uint32_t)(r >> 20) & 0x807F) | ((uint32_t)(120 - e) << 7);
            x[2 * j] = (uint8_t)v;
            x[2 * j + 1] = (uint8_t)(v >> 8);
        } else {
            x[j] = (uint8_t)(((r >> 20) & 0x83) | ((uint32_t)(24 - e) << 2));
        }
    }
    const int nsym = ecf8v_nsym(fmt);
    std::vector<uint64_t> freq(nsym);
    CHECK(ecf8v_histogram(fmt, x.data(), n, freq.data()) == ECF8_OK, "v histogram");
    std::vector<uint8_t> len(ECF8V_MAX_SYM, 0);
    CHECK(ecf8v_code_lengths(freq.data(), nsym, 16, len.data()) == ECF8_OK, "v code lengths");
    ecf8_params p{C, TB};
    ecf8v_meta m;
    CHECK(ecf8v_encode_sizes(fmt, x.data(), n, len.data(), &p, &m) == ECF8_OK, "v sizes");
    std::vector<uint8_t> stream(m.stream_bytes ? m.stream_bytes : 1), raw(m.raw_bytes ? m.raw_bytes : 1),
        gaps(m.gap_bytes ? m.gap_bytes : 1);
    std::vector<uint64_t> blk(m.n_blocks + 1);
    ecf8v_meta m2;
    CHECK(ecf8v_encode(fmt, x.data(), n, len.data(), &p, stream.data(), m.stream_bytes, raw.data(), m.raw_bytes,
                       gaps.data(), m.gap_bytes, blk.data(), m.n_blocks + 1, &m2) == ECF8_OK, "v encode");
    CHECK(ecf8v_validate_meta(&m2) == ECF8_OK, "v validate");
    std::vector<int> olen(nsym);
    for (int s = 0; s < nsym; ++s) olen[s] = len[s];
    const uint64_t T = oraclev_total_bits(fmt, x.data(), n, olen.data());
    uint64_t nc, nb, sb, gb;
    oraclev_sizes(T, C, TB, &nc, &nb, &sb, &gb);
    const uint64_t rb = oraclev_raw_bytes(fmt, n);
    CHECK(T == m.total_bits && sb == m.stream_bytes && rb == m.raw_bytes && gb == m.gap_bytes, "v sizes agree");
    std::vector<uint8_t> os(sb ? sb : 1, 0), orw(rb ? rb : 1, 0), og(gb ? gb : 1, 0);
    std::vector<uint64_t> ob(nb + 1, 0);
    CHECK(oraclev_encode(fmt, x.data(), n, olen.data(), C, TB, os.data(), orw.data(), og.data(), ob.data()) == T,
          "v oracle encode");
    CHECK(std::memcmp(os.data(), stream.data(), sb) == 0 && std::memcmp(orw.data(), raw.data(), rb) == 0 &&
              std::memcmp(og.data(), gaps.data(), gb) == 0 && std::memcmp(ob.data(), blk.data(), 8 * (nb + 1)) == 0,
          "v bytes fmt=%d n=%llu", fmt, (unsigned long long)n);
    std::vector<uint8_t> out(n * eb + 1);
    CHECK(oraclev_decode(fmt, stream.data(), sb, raw.data(), n, olen.data(), out.data()) != (uint64_t)-1, "v decode");
    CHECK(std::memcmp(out.data(), x.data(), n * eb) == 0, "v round trip");
}

int main()
{
    const uint64_t sizes[] = {0, 1, 2, 3, 7, 15, 16, 17, 63, 64, 65, 255, 256, 4095, 4096, 4097, 33333, 100003};
    const uint32_t shapes[][2] = {{16, 256}, {4, 64}, {64, 1024}, {8, 128}};
    int cases = 0;
    for (uint64_t n : sizes)
        for (int kind = 0; kind < 3; ++kind)
            for (auto& sh : shapes) {
                e4m3_case(make_bytes(n, kind), sh[0], sh[1]);
                cases++;
            }
    for (int fmt : {ECF8V_BF16, ECF8V_E5M2})
        for (uint64_t n : {1ull, 17ull, 4097ull, 50001ull})
            for (auto& sh : shapes) {
                variant_case(fmt, n, sh[0], sh[1]);
                cases++;
            }
    // statistics and error strings
    std::vector<float> w(10000);
    for (auto& v : w) v = (float)((double)(next64() >> 11) / 9007199254740992.0 - 0.5);
    double ah = 0;
    CHECK(ecf8_alpha_hat(w.data(), w.size(), 0.01, &ah) == ECF8_OK && ah > 0, "alpha_hat");
    CHECK(ecf8_exponent_entropy_bound(2.0) > 2.66 && ecf8_exponent_entropy_bound(2.0) < 2.67, "entropy bound");
    for (int c = 1; c >= -8; --c) CHECK(ecf8_strerror(c) != nullptr, "strerror %d", c);
    std::printf("%d cases, %d failures\n", cases, g_fail);
    return g_fail ? 1 : 0;
}
