/*
 * ecf8.h -- C ABI of libecf8: lossless ECF8 coding of FP8 E4M3 tensors and
 * their GPU decode on AMD Instinct MI355X (gfx950).
 *
 * ECF8 ("Exponent-Concentrated FP8") keeps every FP8 E4M3 byte bit-exact.
 * The 4-bit exponent field is coded with a per-tensor Huffman code; the sign
 * bit and the 3 mantissa bits stay raw as a packed nibble plane.
 * Sources, cited by page title and section:
 *   - the ECF8 technical blog (codearts.csdn.net), §3.1.1 (per-layer exponent
 *     histogram, optimal prefix code, code length limited to 16 bits), §3.1.2
 *     (table-driven decode), §3.2.1 (chunked parallel decode: each thread owns a
 *     chunk of the bitstream and a stored gap, counts its symbols, a block-wide
 *     reduction places them, threads decode cooperatively into shared memory,
 *     results are written back), §3.2.2 / §3.3 (a preallocated, reused output
 *     pool; batched decode of resident weights), §5.1 (codebook frozen once,
 *     reused at inference);
 *   - the ECF8 paper, "To Compress or Not? Pushing the Frontier of Lossless
 *     GenAI Model Weights Compression with Exponent Concentration"
 *     (arXiv 2510.02676), abstract: the coding is lossless (bit-exact).
 *
 * ------------------------------------------------------------------------
 * Encoded format (one tensor of n elements; C = chunk_bytes, TB = lanes per
 * block).  The pages fix the method, not the byte layout; the layout below is
 * this library's reading and both the encoder and decoder obey it exactly.
 *   symbol      e_j = (x_j >> 3) & 15           (raw exponent field, 0..15)
 *   code        canonical Huffman: symbols sorted by (length, symbol), first
 *               code 0, next = (prev + 1) << (length growth); lengths 1..16
 *   stream      codes of e_0..e_{n-1} concatenated MSB-first: stream bit k is
 *               bit 7 - (k % 8) of byte k / 8.  T = total code bits.
 *               n_chunks = ceil(T / 8C), n_blocks = ceil(n_chunks / TB);
 *               stream_bytes = n_blocks*TB*C + 16, zero padded.
 *   nibbles     nib_j = ((x_j >> 7) << 3) | (x_j & 7) in byte j/2, low nibble
 *               for even j; nibble_bytes = ceil(n / 16) * 8, zero padded.
 *   gaps        chunk t covers stream bits [8Ct, 8C(t+1)).  gap_t = first
 *               codeword start p >= 8Ct (with T counted as a start) minus 8Ct,
 *               for 8Ct < T; 0 for chunks at or past T.  Always in 0..15.
 *               Two per byte, low nibble for even t; gap_bytes = n_blocks*TB/2.
 *   blk_off     uint64[n_blocks + 1]; blk_off[b] = number of codewords that
 *               start before bit 8*C*TB*b; blk_off[n_blocks] = n.
 * Decoded byte: x_j = ((nib_j >> 3) << 7) | (e_j << 3) | (nib_j & 7).
 * ------------------------------------------------------------------------
 *
 * Conventions: every function returns ECF8_OK (0) or a negative ECF8_ERR_*.
 * The caller owns every buffer.  Host functions take host pointers; decode
 * functions take device pointers (HIP device memory) and run asynchronously
 * on the given hipStream_t (passed as void*; NULL = the null stream).  The
 * decode entry points allocate no device memory: scratch space is the
 * caller's workspace, or, for ecf8_decode_batched_noalloc, a fixed device
 * array of the library.
 */
#ifndef ECF8_H
#define ECF8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ECF8_NSYM 16          /* exponent symbols of FP8 E4M3 */
#define ECF8_MAX_CODE_LEN 16  /* ECF8 blog §3.1.1: code length limited to 16 bits */

enum {
    ECF8_OK = 0,
    ECF8_ERR_ARG = -1,          /* NULL / misaligned pointer, bad count or parameter */
    ECF8_ERR_SIZE = -2,         /* n or a buffer capacity disagrees with the metadata */
    ECF8_ERR_META = -3,         /* metadata fails validation */
    ECF8_ERR_UNSUPPORTED = -4,  /* valid parameters with no decode kernel, or a length
                                   limit below the Huffman depth */
    ECF8_ERR_CORRUPT = -5,      /* decode found symbol counts that disagree with blk_off */
    ECF8_ERR_HIP = -6,          /* HIP runtime error */
    ECF8_ERR_WORKSPACE = -7     /* workspace NULL, misaligned or too small */
};

/* Code lengths per exponent symbol (0 = symbol absent).  ECF8 blog §3.1.1. */
typedef struct {
    uint8_t len[ECF8_NSYM];
} ecf8_codebook;

/* Chunk bytes per lane (C) and lanes per block (TB).  ECF8 blog §3.2.1 / §5.2
 * describe 64-byte per-thread chunks and 128-thread blocks on their hardware;
 * here they are format parameters.  Encode accepts C in {4,8,...,64}
 * (multiple of 4) and TB in {64,128,...,1024} (multiple of 64).  Decode
 * kernels exist for (C, TB) = (16, 256) (the tuned shape), (32, 256),
 * (64, 128) (the pages' shape), (16, 128), (8, 256) and (16, 512); other
 * pairs decode with ECF8_ERR_UNSUPPORTED.  All tensors of one batched decode
 * share one shape (ECF8_ERR_UNSUPPORTED otherwise). */
typedef struct {
    uint32_t chunk_bytes;
    uint32_t threads_per_block;
} ecf8_params;

/* Everything the decoder needs besides the four buffers. */
typedef struct {
    uint64_t n;             /* elements */
    uint64_t total_bits;    /* T */
    uint64_t n_chunks;
    uint64_t n_blocks;
    uint64_t stream_bytes;
    uint64_t nibble_bytes;
    uint64_t gap_bytes;
    uint32_t chunk_bytes;
    uint32_t threads_per_block;
    ecf8_codebook cb;
    uint32_t max_len;       /* longest code length in cb (0 when n = 0) */
    uint32_t reserved;
} ecf8_meta;

/* The four encoded buffers of one tensor.  Device pointers when decoding.
 * Alignment required by decode: stream 16 B, nibbles 8 B, blk_off 8 B. */
typedef struct {
    const uint8_t* stream;
    const uint8_t* nibbles;
    const uint8_t* gaps;
    const uint64_t* blk_off;
} ecf8_stream;

/* One tensor of a batched decode: its buffers, metadata and the byte offset of
 * its output inside out_base (must keep the output 16-byte aligned). */
typedef struct {
    ecf8_stream s;
    ecf8_meta meta;
    uint64_t out_offset;
} ecf8_tensor_desc;

/* A prepared batched decode (host struct, filled by ecf8_decode_prepare). */
typedef struct {
    void* workspace;
    uint64_t workspace_bytes;
    uint64_t total_blocks;
    uint32_t count;
    uint32_t chunk_bytes;
    uint32_t threads_per_block;
    uint32_t grid;           /* workgroups of the persistent decode kernel; the caller
                                may lower it (to any value >= 1) before a run to leave
                                compute units to kernels on other streams: every
                                workgroup walks blocks grid apart, so all blocks are
                                decoded whatever the value */
    uint32_t short_codes;    /* 1: every tensor's code is complete with no codeword longer
                                than 11 bits, and the decode indexes its tables with the
                                11-bit prefix alone (set by ecf8_decode_prepare; a tensor
                                that does not qualify is not decoded under 1 and its blocks
                                are counted by ecf8_decode_status) */
    uint32_t claim_blocks;   /* block order of a run.  0: workgroup g decodes blocks g,
                                g + grid, g + 2 grid, ...  k (2..1024): workgroups take
                                claims of k consecutive blocks, the first one each by
                                its index and the rest from a counter in the workspace,
                                which keeps the blocks in flight close together over a
                                long dispatch.  ecf8_decode_prepare sets 4 when the
                                plan has at least 64 blocks per workgroup, else 0; the
                                caller may change it before a run (total_blocks + grid *
                                claim_blocks must stay below 2^32).  Runs of one plan
                                must not overlap in time: they share the counter */
} ecf8_plan;

/* ---------------------------- host side ------------------------------- */

/* ECF8 blog §3.1.1 step 1: histogram of the exponent field of n FP8 bytes.
 * fp8: host, n bytes; freq: host, 16 counters (overwritten).
 * Errors: ECF8_ERR_ARG if fp8 is NULL with n > 0 or freq is NULL. */
int ecf8_histogram(const uint8_t* fp8, uint64_t n, uint64_t freq[ECF8_NSYM]);

/* ECF8 blog §3.1.1 steps 2-3: Huffman code lengths from a histogram, ties
 * broken on (weight, node id) with leaves numbered by symbol and merged nodes
 * numbered 16, 17, ... in creation order; one present symbol gets length 1.
 * max_len: the length limit, 1..16 (a 16-symbol Huffman tree is at most 15
 * deep, so 15 and 16 never bind).  When the Huffman code is deeper than
 * max_len, the lengths are the optimal ones no longer than max_len
 * (package-merge, as ecf8v_code_lengths).  A limit of 11 or less lets the
 * decode index its tables with one shift (ecf8_plan.short_codes).
 * ECF8_ERR_UNSUPPORTED if 2^max_len is below the number of present symbols.
 * out: host. */
int ecf8_codebook_from_freq(const uint64_t freq[ECF8_NSYM], uint32_t max_len, ecf8_codebook* out);

/* ecf8_histogram + ecf8_codebook_from_freq ("build once, freeze", ECF8 blog §5.1). */
int ecf8_build_codebook(const uint8_t* fp8, uint64_t n, uint32_t max_len, ecf8_codebook* out);

/* Canonical codes of a codebook (MSB-first values, length in cb->len). */
int ecf8_canonical_codes(const ecf8_codebook* cb, uint32_t code[ECF8_NSYM]);

/* Size query for ECF8 blog §3.1.1 (the exponent stream T = sum of code
 * lengths) and §3.2.1 (the stream cut into per-thread chunks of C bytes, each
 * with a stored gap, and blocks of TB threads): fills *out (T, chunk/block
 * counts, the four buffer sizes) for encoding fp8 with cb and params.
 * fp8: host, n bytes (not modified); out: host, overwritten.
 * Errors: ECF8_ERR_META if an element's exponent has length 0 in cb or cb is
 * not a prefix code; ECF8_ERR_ARG on NULL pointers or bad params. */
int ecf8_encode_sizes(const uint8_t* fp8, uint64_t n, const ecf8_codebook* cb,
                      const ecf8_params* params, ecf8_meta* out);

/* ECF8 blog §3.1.1 / §3.2.1: encode n FP8 bytes (host) into the stream,
 * nibble plane, gaps and block offsets (host buffers of at least the sizes
 * ecf8_encode_sizes reports, in bytes; blk_cap counts uint64 entries).  Every
 * byte of the four buffers is written (padding zeroed).  Multithreaded.
 * Errors as ecf8_encode_sizes, ECF8_ERR_SIZE if a capacity is too small. */
int ecf8_encode(const uint8_t* fp8, uint64_t n, const ecf8_codebook* cb, const ecf8_params* params,
                uint8_t* stream, uint64_t stream_cap, uint8_t* nibbles, uint64_t nibble_cap,
                uint8_t* gaps, uint64_t gap_cap, uint64_t* blk_off, uint64_t blk_cap,
                ecf8_meta* meta);

/* ECF8 blog §5.3 (troubleshooting: wrong output -> check that the gap values
 * agree with the stream): the host-side part of that check, a structural
 * check of metadata before any decode: sizes consistent with n, T, C, TB
 * (§3.2.1 chunk and block counts); code lengths 0..16 forming a prefix code
 * (§3.1.1: optimal prefix code, at most 16 bits; Kraft sum 1 with >= 2
 * symbols, one symbol of length 1 otherwise); max_len correct.  meta: host,
 * read only.  Returns ECF8_OK, or ECF8_ERR_META (ECF8_ERR_ARG if NULL). */
int ecf8_validate_meta(const ecf8_meta* meta);

/* -------------------------- device decode ----------------------------- */

/* Workspace bytes a decode of `count` tensors needs (256-byte aligned
 * device memory, owned by the caller, sized once and reused across calls, as
 * ECF8 blog §3.2.2 sizes its pool once): a 256-byte status area (the
 * block-check counter, and at byte 64 the claimed block order's two counters),
 * 144 bytes of descriptor per tensor (rounded up to a multiple of 256 in
 * all) and 9,216 bytes of decode table per tensor.  Returns 0 for
 * count < 0. */
uint64_t ecf8_workspace_bytes(int count);

/* Batched-decode setup (ECF8 blog §3.3, "resident weights + batched decode"):
 * validates every descriptor on the host, writes the device descriptor table
 * into the workspace (one small host-to-device copy on hip_stream), launches
 * on hip_stream the table kernel that builds each tensor's canonical decode
 * table from its 16 code lengths into the workspace (ECF8 blog §3.1.2; once
 * per plan, since a tensor's codebook does not change) and fills *plan.  The
 * workspace's block-check counter starts at 0.  All tensors must share
 * (C, TB).  out_base: device, receives tensor i
 * at out_base + descs[i].out_offset (n_i bytes).  The plan stays valid while
 * the workspace and the tensors' buffers do.
 * Errors: ECF8_ERR_ARG/SIZE/META/UNSUPPORTED/WORKSPACE/HIP. */
int ecf8_decode_prepare(const ecf8_tensor_desc* descs, int count, uint8_t* out_base,
                        void* workspace, uint64_t workspace_bytes, void* hip_stream,
                        ecf8_plan* plan);

/* One batched decode of a prepared plan: one persistent dispatch over every
 * block of every tensor, running the ECF8 blog §3.2.1 phases on each block
 * (chunk load, gap-based symbol count, block-wide exclusive scan,
 * cooperative decode into LDS, coalesced write-back) with the decode table
 * of the block's tensor (ECF8 blog §3.1.2, built by ecf8_decode_prepare)
 * copied into LDS by each workgroup when its tensor changes.  Must follow the
 * plan's ecf8_decode_prepare on the same stream, or on a stream ordered
 * after it.  Asynchronous on hip_stream; the return code covers launch errors
 * only (ECF8_ERR_ARG/WORKSPACE/HIP). */
int ecf8_decode_run(const ecf8_plan* plan, void* hip_stream);

/* For measurement (the pages time the decode as a whole, ECF8 blog §4; this
 * times the kernel): ecf8_decode_run with HIP events attached to the
 * dispatch itself, so that they hold its start and end times (hipEvent_t
 * handles created by the caller with timing enabled; either may be NULL).
 * Events recorded on the stream around an ordinary launch also hold the
 * dispatch's launch and completion latency.  Same errors as
 * ecf8_decode_run. */
int ecf8_decode_run_timed(const ecf8_plan* plan, void* hip_stream, void* start_event, void* stop_event);

/* ECF8 blog §3.3 (data-centre mode: every weight resident, decoded in
 * batches) and §3.2.2 (one preallocated output pool, reused, no allocation);
 * DFloat11 blog §3.3 (the weights of a whole transformer block decoded
 * together): decode `count` tensors in one persistent dispatch into
 * out_base (tensor i at out_base + descs[i].out_offset, n_i bytes, 16-byte
 * aligned, ranges must not overlap).  = ecf8_decode_prepare +
 * ecf8_decode_run.  descs: host, read during the call only; buffers and
 * workspace: device, caller-owned.  Asynchronous on hip_stream.
 * Errors: those of ecf8_decode_prepare and ecf8_decode_run. */
int ecf8_decode_batched(const ecf8_tensor_desc* descs, int count, uint8_t* out_base,
                        void* workspace, uint64_t workspace_bytes, void* hip_stream);

/* ECF8 blog §3.2.1, the decode kernel of one bitstream and its metadata
 * (per-thread chunk load, gap-based symbol count, block-wide scan,
 * cooperative decode into shared memory, write-back): decode one tensor.
 * s: host struct of device pointers (stream 16-byte aligned, nibbles and
 * blk_off 8-byte aligned); meta: host; out_fp8: device, 16-byte aligned,
 * receives exactly n bytes; n must equal meta->n (ECF8_ERR_SIZE otherwise).
 * workspace: device, >= ecf8_workspace_bytes(1) bytes, 256-byte aligned,
 * caller-owned (descriptor, decode table and block-check counter; the
 * library allocates nothing).  Equivalent to ecf8_decode_batched with
 * count = 1.  Asynchronous on hip_stream; the return code covers argument
 * and metadata checks and launch errors (ECF8_ERR_ARG/SIZE/META/
 * UNSUPPORTED/WORKSPACE/HIP). */
int ecf8_decode(const ecf8_stream* s, const ecf8_meta* meta, uint8_t* out_fp8, uint64_t n,
                void* workspace, uint64_t workspace_bytes, void* hip_stream);

/* Checked mode, after ECF8 blog §5.3 (wrong output -> verify the gap
 * synchronisation): every decoded block compares the sum of its threads'
 * symbol counts (each counted from the thread's stored gap) with its stored
 * offsets blk_off[b + 1] - blk_off[b].  This call synchronizes hip_stream,
 * reads the workspace's counter of disagreeing blocks into *bad_blocks
 * (host), restarts it, and returns ECF8_ERR_CORRUPT if it was non-zero.  The
 * counter covers every run on the workspace since ecf8_decode_prepare wrote
 * it (cleared) or since the previous call of this function.  A corrupt stream, gap or offset that keeps every block's
 * count is not detected (the format carries no checksum); whatever the
 * corruption, no byte outside each tensor's output range is written.
 * Errors: ECF8_ERR_ARG (NULL), ECF8_ERR_HIP. */
int ecf8_decode_status(const void* workspace, void* hip_stream, uint64_t* bad_blocks);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc): the same
 * decode as ecf8_decode_batched, with no workspace argument.  Its block-check
 * counter, descriptors and decode tables live in a fixed device array of the
 * library, 150,016 bytes per GPU, held by each GPU the library runs on until
 * the process ends; it holds at most 16 tensors (count > 16 returns
 * ECF8_ERR_WORKSPACE).  The descriptors reach the device as kernel arguments,
 * so the call allocates nothing, copies nothing and issues no memset:
 * launches only (a setup kernel per 8 tensors, the table kernel, the decode).
 * Every call on one GPU shares that array: calls that overlap on one GPU (on
 * different streams, unordered) race and must not be issued; calls ordered on
 * one stream are safe (each rewrites what it uses).  bad_blocks: NULL, or a
 * device uint64 (8-byte aligned, caller-owned) that receives the number of
 * blocks whose symbol count disagreed with blk_off (checked mode; zeroed at
 * the start of each call, complete when the stream reaches the end of the
 * decode).  Other arguments, alignment and errors as ecf8_decode_batched.
 * Asynchronous on hip_stream. */
int ecf8_decode_batched_noalloc(const ecf8_tensor_desc* descs, int count, uint8_t* out_base,
                                uint64_t* bad_blocks, void* hip_stream);

/* ---------------------------- device encode ---------------------------- */

/* ECF8 blog §3.1.1 step 1 on the GPU: histogram of the exponent field of n
 * FP8 E4M3 bytes.  fp8: device; freq: device, 16 uint64 counters (8-byte
 * aligned), overwritten.  workspace: NULL, or device memory of at least
 * ecf8_encode_workspace_bytes(n) bytes (256-byte aligned, caller-owned) that
 * receives the per-tile symbol counts ecf8_encode_device needs for the same
 * data.  Asynchronous on hip_stream.
 * Errors: ECF8_ERR_ARG (NULL or misaligned), ECF8_ERR_WORKSPACE, ECF8_ERR_HIP. */
int ecf8_histogram_device(const uint8_t* fp8, uint64_t n, uint64_t* freq, void* workspace,
                          uint64_t workspace_bytes, void* hip_stream);

/* Host: metadata (T = sum of freq[s] * len[s], chunk and block counts, the
 * four buffer sizes) for n elements with exponent histogram freq, codebook cb
 * and params -- what ecf8_encode_sizes computes, without the data.
 * Errors as ecf8_encode_sizes. */
int ecf8_meta_from_freq(const uint64_t freq[ECF8_NSYM], uint64_t n, const ecf8_codebook* cb,
                        const ecf8_params* params, ecf8_meta* out);

/* Device workspace bytes ecf8_histogram_device and ecf8_encode_device need
 * for n elements (256-byte aligned device memory, owned by the caller):
 * 32 B per 4096 elements of per-tile counts, 8 B per 4096 of tile offsets. */
uint64_t ecf8_encode_workspace_bytes(uint64_t n);

/* ECF8 blog §3.1.1 / §3.2.1 on the GPU: encode n = meta->n FP8 bytes (fp8,
 * device) into the four device buffers, of at least meta's sizes: the same
 * bytes as ecf8_encode writes (canonical codes MSB-first, nibble plane, gaps,
 * block offsets, padding zeroed).  workspace: the one ecf8_histogram_device
 * filled for this same data (it holds the per-tile symbol counts, which fix
 * every tile's bit offset; the counts are kept, so one histogram serves
 * several encodes of the data under different codes or parameters).  meta
 * comes from ecf8_meta_from_freq (or ecf8_encode_sizes) for this data and is
 * validated.  Counts or a meta that do not match the data give a wrong
 * stream, which fails decode's block check, but no write leaves the four
 * buffers or the workspace.  n = 0 writes the 16 zero bytes of the stream and
 * blk_off[0] = 0 only (fp8, nibbles, gaps and workspace may be NULL).
 * Alignment: stream and gaps 4 B, nibbles and blk_off 8 B, workspace 256 B.
 * Asynchronous on hip_stream: two scan launches (group totals, tile
 * offsets), the encode, and one launch for the words two encode workgroups
 * share.  The same as ecf8_encode_batched_device with one job.
 * Errors: ECF8_ERR_ARG (NULL or misaligned), ECF8_ERR_META,
 * ECF8_ERR_WORKSPACE, ECF8_ERR_SIZE (n >= 2^37), ECF8_ERR_HIP. */
int ecf8_encode_device(const uint8_t* fp8, const ecf8_meta* meta, uint8_t* stream, uint8_t* nibbles,
                       uint8_t* gaps, uint64_t* blk_off, void* workspace, uint64_t workspace_bytes,
                       void* hip_stream);

/* One tensor of ecf8_encode_batched_device: the arguments of
 * ecf8_encode_device, with the metadata by value. */
typedef struct {
    const uint8_t* fp8;        /* device, meta.n bytes */
    ecf8_meta meta;            /* from ecf8_meta_from_freq (or ecf8_encode_sizes) for this data */
    uint8_t* stream;           /* device outputs of at least meta's sizes */
    uint8_t* nibbles;
    uint8_t* gaps;
    uint64_t* blk_off;
    void* workspace;           /* the workspace ecf8_histogram_device filled for this data */
    uint64_t workspace_bytes;
} ecf8_encode_job;

/* ECF8 blog §3.1.1 / §3.2.1 on the GPU, for several tensors at once (a
 * layer re-encoded after its weights change, DFloat11 §5 "dynamic codebook
 * update"): jobs[0 .. count) encoded as ecf8_encode_device would encode each
 * (same bytes, same alignment and workspace rules), eight tensors per set of
 * four launches instead of four launches per tensor.  jobs is host memory,
 * read before the call returns; the tensors' buffers must not overlap.  Every
 * job is checked before anything is launched: on an error nothing is
 * written.  Asynchronous on hip_stream.
 * Errors: ECF8_ERR_ARG (count < 0, jobs NULL with count > 0, or a job's
 * pointers NULL or misaligned), and per job as ecf8_encode_device. */
int ecf8_encode_batched_device(const ecf8_encode_job* jobs, int count, void* hip_stream);

/* ------------------------- weight statistics --------------------------- */

/* ECF8 blog §6 (adaptive α estimation): the tail-index estimate
 *     α̂ = log n / log(max_i |w_i| / γ)
 * of n weights w (host, float32, before FP8 quantization) of an α-stable law
 * with scale γ.  NaN weights are skipped.  *alpha_hat receives α̂ (natural
 * logs; the ratio makes the base irrelevant).
 * Errors: ECF8_ERR_ARG if w is NULL with n > 0, alpha_hat is NULL, n < 2,
 * γ <= 0 (or NaN), or max |w| <= γ (the estimate is then undefined). */
int ecf8_alpha_hat(const float* w, uint64_t n, double gamma, double* alpha_hat);

/* ECF8 blog §2.2: the upper bound α / (1 - 2^-α) on the entropy, in bits, of
 * the floating-point exponent of an α-stable weight (8/3 at α = 2).  NaN for
 * α <= 0. */
double ecf8_exponent_entropy_bound(double alpha);

/* ------------------------------ measurement ------------------------------ */

/* A plain streaming copy of `bytes` bytes from src to dst (device memory,
 * both 16-byte aligned, not overlapping): dwordx4 loads and stores, four in
 * flight per lane, non-temporal hints, a persistent grid of 8 workgroups per
 * compute unit.  It is not part of the method: the decode is bound by HBM
 * traffic, and this copy is the ceiling its traffic is compared with (its
 * rate, and the FETCH_SIZE / WRITE_SIZE counters it reads for a known size,
 * calibrate the decode's measurements).  Asynchronous on hip_stream.
 * Errors: ECF8_ERR_ARG (NULL or misaligned with bytes > 0), ECF8_ERR_HIP. */
int ecf8_hbm_copy(const void* src, void* dst, uint64_t bytes, void* hip_stream);

/* A plain stream with a decode's byte mix: write_bytes to dst while reading
 * read_bytes (<= write_bytes) from src, each byte once: output 16-byte unit i
 * takes input unit (i * m) >> 32, m = floor(2^32 * read_units / write_units),
 * so neighbouring lanes share input units and their cache lines.  Same grid,
 * loads, stores and hints as ecf8_hbm_copy.  Not part of the method: the rate
 * a decode moving the same bytes could reach with no work of its own (a
 * tighter ceiling than the copy, whose reads and writes are equal).  Both
 * sizes multiples of 16, both pointers 16-byte aligned, write_bytes / 16 <
 * 2^32.  Asynchronous on hip_stream.
 * Errors: ECF8_ERR_ARG (NULL, misaligned, sizes not multiples of 16, read
 * 0 or more than written), ECF8_ERR_SIZE, ECF8_ERR_HIP. */
int ecf8_hbm_stream(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes, void* hip_stream);

/* Human-readable name of an error code (static string). */
const char* ecf8_strerror(int code);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int ecf8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ECF8_H */
