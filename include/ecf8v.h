/*
 * ecf8v.h -- C ABI of libecf8 for the exponent-coding variants of two more
 * float formats, with their GPU decode on AMD Instinct MI355X (gfx950):
 *   ECF8V_BF16  BFloat16, the DFloat11 layout: the 8-bit exponent is coded
 *               (256 symbols), sign and 7 mantissa bits stay raw;
 *   ECF8V_E5M2  FP8 E5M2: the 5-bit exponent is coded (32 symbols), sign and
 *               2 mantissa bits stay raw.
 * Sources, cited by page title and section:
 *   - the DFloat11 article (BFloat16 weights), §2 (per-tensor exponent
 *     statistics, Huffman codes for the exponent, sign and mantissa kept),
 *     §3.2 (exponents decoded cooperatively per block, floats reassembled),
 *     §3.3 (a transformer block's weights decoded together);
 *   - the ECF8 technical blog (codearts.csdn.net), §3.1.1 (code length
 *     limited to 16 bits) and §3.2.1 (per-lane chunks with stored gaps,
 *     counts, block scan, cooperative decode, write back).
 * With 256 symbols the Huffman depth can pass 16, so the code lengths come
 * from an optimal length-limited construction (package-merge: Larmore and
 * Hirschberg, J. ACM 37(3), 1990).
 *
 * ------------------------------------------------------------------------
 * Encoded format: the E4M3 format of ecf8.h (canonical codes in (length,
 * symbol) order, MSB-first stream, chunk gaps, block offsets, the same sizes)
 * with a wider symbol and a different raw plane:
 *   BF16  value v (uint16, little-endian in memory): symbol (v >> 7) & 255;
 *         raw byte (sign << 7) | (v & 127), one byte per element;
 *         raw_bytes = ceil(n / 16) * 16.
 *         Decoded v = ((raw >> 7) << 15) | (symbol << 7) | (raw & 127).
 *   E5M2  byte b: symbol (b >> 2) & 31; raw nibble (sign << 2) | (b & 3) in
 *         the E4M3 nibble layout (element j in byte j / 2, low nibble for even
 *         j); raw_bytes = ceil(n / 16) * 8.
 *         Decoded b = ((raw >> 2) << 7) | (symbol << 2) | (raw & 3).
 * Code lengths are at most 16 (gaps stay in 0..15).
 * ------------------------------------------------------------------------
 * Conventions as in ecf8.h: ECF8_OK or a negative ECF8_ERR_*; the caller owns
 * every buffer; host functions take host pointers, decode functions device
 * pointers and a hipStream_t passed as void*.
 */
#ifndef ECF8V_H
#define ECF8V_H

#include <stdint.h>

#include "ecf8.h"

#ifdef __cplusplus
extern "C" {
#endif

#define ECF8V_BF16 1
#define ECF8V_E5M2 2
#define ECF8V_MAX_SYM 256

/* Everything the decoder needs besides the four buffers. */
typedef struct {
    uint64_t n;               /* elements */
    uint64_t total_bits;      /* T */
    uint64_t n_chunks;
    uint64_t n_blocks;
    uint64_t stream_bytes;
    uint64_t raw_bytes;
    uint64_t gap_bytes;
    uint32_t chunk_bytes;
    uint32_t threads_per_block;
    uint32_t format;          /* ECF8V_BF16 or ECF8V_E5M2 */
    uint32_t max_len;         /* longest code length (0 when n = 0) */
    uint8_t len[ECF8V_MAX_SYM];   /* code length per symbol; entries past the
                                     format's symbol count are 0 */
} ecf8v_meta;

/* Symbols of a format (256 for BF16, 32 for E5M2), or ECF8_ERR_ARG. */
int ecf8v_nsym(uint32_t format);

/* DFloat11 article §2 step 1: histogram of the exponent field.  data: host,
 * n elements of the format (BF16: uint16 values; E5M2: bytes); freq: host,
 * ecf8v_nsym(format) counters (overwritten).  Errors: ECF8_ERR_ARG. */
int ecf8v_histogram(uint32_t format, const void* data, uint64_t n, uint64_t* freq);

/* Optimal prefix-code lengths no longer than max_len (1..16) for the counts
 * freq[0..nsym) (nsym <= 256), by package-merge: the least total coded bits
 * among all prefix codes with lengths <= max_len.  Absent symbols get 0, a
 * single present symbol 1.  len: host, nsym entries.
 * Errors: ECF8_ERR_ARG (NULL, nsym or max_len out of range),
 * ECF8_ERR_UNSUPPORTED (2^max_len < present symbols). */
int ecf8v_code_lengths(const uint64_t* freq, uint32_t nsym, uint32_t max_len, uint8_t* len);

/* Canonical codes (MSB-first values) of lengths len[0..nsym); returns
 * ECF8_ERR_META if a length passes 16 or the lengths over-fill the code. */
int ecf8v_canonical_codes(const uint8_t* len, uint32_t nsym, uint32_t* code);

/* Sizes and T for encoding data with lengths len (nsym entries of the
 * format) and params.  Errors: ECF8_ERR_ARG, ECF8_ERR_META (a present symbol
 * without a code, or bad lengths). */
int ecf8v_encode_sizes(uint32_t format, const void* data, uint64_t n, const uint8_t* len,
                       const ecf8_params* params, ecf8v_meta* out);

/* DFloat11 article §2 / ECF8 blog §3.2.1: encode n elements into host
 * buffers of at least the sizes ecf8v_encode_sizes gives (stream, raw, gaps:
 * bytes; blk_off: n_blocks + 1 entries); *meta is filled.
 * Errors: as ecf8v_encode_sizes, ECF8_ERR_SIZE (a capacity too small). */
int ecf8v_encode(uint32_t format, const void* data, uint64_t n, const uint8_t* len, const ecf8_params* params,
                 uint8_t* stream, uint64_t stream_cap, uint8_t* raw, uint64_t raw_cap, uint8_t* gaps,
                 uint64_t gap_cap, uint64_t* blk_off, uint64_t blk_cap, ecf8v_meta* meta);

/* 0 if the metadata is self-consistent, else ECF8_ERR_META. */
int ecf8v_validate_meta(const ecf8v_meta* meta);

/* One tensor of a batched variant decode: its buffers (device), metadata and
 * the byte offset of its output inside out_base (16-byte aligned). */
typedef struct {
    const uint8_t* stream;
    const uint8_t* raw;
    const uint8_t* gaps;
    const uint64_t* blk_off;
    ecf8v_meta meta;
    uint64_t out_offset;
} ecf8v_tensor_desc;

/* A prepared batched variant decode (host struct). */
typedef struct {
    void* workspace;
    uint64_t workspace_bytes;
    uint64_t total_blocks;
    uint32_t count;
    uint32_t format;
    uint32_t threads_per_block;
    uint32_t grid;            /* persistent workgroups; may be lowered (>= 1) */
    uint32_t table_entries;   /* LDS decode-table entries: the plan's largest table */
    uint32_t short_codes;     /* 1: no code of the batch is longer than 10 bits, and the decode
                                 indexes its tables with one shift (chosen by ecf8v_decode_prepare) */
} ecf8v_plan;

/* Device workspace bytes for a batched decode of `count` tensors (256-byte
 * aligned device memory, owned by the caller). */
uint64_t ecf8v_workspace_bytes(int count);

/* Validate `count` descriptors of one format, upload them to the workspace
 * and build every tensor's decode table there (on hip_stream, waited for: the
 * tables depend on the code lengths only).  A table has one entry per 10-bit
 * prefix covered by codewords of at most 10 bits and one per 16-bit value of
 * the space the longer codewords take (at most 9089 entries for any valid
 * code); each entry decodes up to three whole codewords.  Decode kernels
 * exist for chunk_bytes = 16 and threads_per_block in {64, 128, 256}; other
 * params give ECF8_ERR_UNSUPPORTED.  Output of tensor i: out_base +
 * out_offset_i, n_i elements of the format.  Errors: ECF8_ERR_ARG,
 * ECF8_ERR_META, ECF8_ERR_UNSUPPORTED, ECF8_ERR_WORKSPACE, ECF8_ERR_HIP. */
int ecf8v_decode_prepare(const ecf8v_tensor_desc* descs, int count, uint8_t* out_base, void* workspace,
                         uint64_t workspace_bytes, void* hip_stream, ecf8v_plan* plan);

/* DFloat11 article §3.2 / ECF8 blog §3.2.1: the decode of a prepared plan,
 * asynchronous on hip_stream: one persistent dispatch over all tensors'
 * blocks (the workspace must still hold what prepare put there).  Errors:
 * ECF8_ERR_ARG (NULL plan or workspace, grid 0, a bad table size),
 * ECF8_ERR_UNSUPPORTED, ECF8_ERR_HIP (launch). */
int ecf8v_decode_run(const ecf8v_plan* plan, void* hip_stream);

/* For measurement: ecf8v_decode_run with HIP events attached to the
 * dispatch itself (hipEvent_t handles created by the caller with timing
 * enabled; either may be NULL), so that they hold its start and end times.
 * Same errors as ecf8v_decode_run. */
int ecf8v_decode_run_timed(const ecf8v_plan* plan, void* hip_stream, void* start_event, void* stop_event);

/* Synchronize hip_stream and report the blocks whose decoded symbol count
 * disagreed with blk_off, or whose stream held a window that is no codeword
 * (those blocks are not written), in *bad_blocks; returns ECF8_ERR_CORRUPT
 * if non-zero.  The count covers every run on the workspace since
 * ecf8v_decode_prepare cleared it or since the previous call of this
 * function, which restarts it. */
int ecf8v_decode_status(const void* workspace, void* hip_stream, uint64_t* bad_blocks);

#ifdef __cplusplus
}
#endif

#endif /* ECF8V_H */
