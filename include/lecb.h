/*
 * lecb.h -- C ABI of the MI355X (gfx950) Huffman byte codec.
 *
 * What it computes
 * ----------------
 * Lossless Huffman coding of 8-bit tensor symbols, two ways:
 *
 *  - fixed-codebook, single-stage coding ("Single-Stage Huffman Encoder for
 *    ML Compression", Methodology steps 1-4): symbol statistics of a few
 *    warm-up batches are summed, one canonical codebook is built from them
 *    once and kept on the device, and every later tensor is coded with it
 *    directly -- no per-tensor histogram, no codebook in the stream;
 *
 *  - byte-grouped, per-tensor coding of bf16 tensors ("Lossless Compression
 *    for LLM Tensor Incremental Snapshots", Technical framework steps 1-3 and
 *    the reverse path): the 16-bit words are split into a high-byte and a
 *    low-byte plane, each plane gets its own histogram and its own codebook,
 *    and decoding restores the 16-bit words.  32-bit elements (fp32) are
 *    grouped the same way into four byte planes (the byte-group size is a
 *    design knob of the same page, Key design item 1).
 *
 * Stream format v3 (identical, bit for bit, to the oracle's):
 *   stream  = u32 end[nc] | zero pad to 16 B | u16 nw[nc*G] | zero pad to 16 B | u32 payload[W]
 *   nc      = ceil(n / chunk); chunk c holds symbols [c*chunk, min((c+1)*chunk, n));
 *   lanes   = G = min(chunk/256, 16) per chunk: the chunk's blocks of 16
 *             symbols (the last one shorter) go round-robin to the lanes,
 *             block b to lane b mod G;
 *   lane    = its symbols' code words concatenated, most significant bit
 *             first, in 32-bit words, the last one zero-padded; nw[c*G + j]
 *             = the words of lane j of chunk c (0 for a lane with no symbols);
 *   payload = per chunk, its lanes' words in the order a lane-parallel
 *             decoder reads them: every lane's word 0, then every lane's
 *             word 1 (lane order, only words that exist), then, pair of
 *             symbols by pair, a lane's word k >= 2 just before its first pair
 *             that starts at or after bit 32(k-1) of the lane (lane order
 *             within a pair); words stored little-endian;
 *   end[c]  = payload word one past chunk c's last word (chunk c spans
 *             [end[c-1], end[c]) with end[-1] = 0); W = end[nc-1];
 *   size    = align16(4*nc) + align16(2*nc*G) + 4*W  (0 when n == 0).
 * The lanes are the independent parallel tasks of "Lossless Compression for
 * LLM Tensor Incremental Snapshots", Key design item 3; the layout is this
 * library's choice (the pages fix none): lanes of a chunk write neighbouring
 * output blocks and read one shared, sequential word stream.
 * The codebook is not in the stream.  Code words are canonical: they follow
 * from the 256 code lengths alone (shorter codes first, ties by symbol).
 *
 * Conventions
 * -----------
 *  - Every buffer is owned by the caller.  Device pointers are HIP device
 *    memory on the current device, 16-byte aligned.  `stream` arguments are
 *    hipStream_t passed as void* (NULL = the null stream).
 *  - Device entry points only enqueue work on `stream`; they never
 *    synchronise and never allocate.  The exceptions are the entries that
 *    build a codebook from the tensor itself (lecb_encode_bf16_pertensor,
 *    lecb_encode_bf16_delta_pertensor, lecb_encode_fp32_pertensor,
 *    lecb_encode_adaptive): they read the histograms back, which
 *    synchronises `stream` once, and on their first call in a host thread
 *    allocate an 8 KiB pinned host buffer that the thread keeps.
 *  - Return values: LECB_OK or a negative lecb_status detected on the host
 *    (bad argument, too small a buffer).  Problems only the GPU can see
 *    (a byte with no code word, a corrupt stream, output overflow) are
 *    written to lecb_result.status in device memory; read it after
 *    synchronising.  On any error the output contents are undefined.
 *  - A workspace (lecb_workspace_bytes) must be zero-filled once, e.g. with
 *    lecb_workspace_init, before its first use.  Every call leaves it ready
 *    for the next.  Calls that overlap in time must not share a workspace.
 *  - chunk must be a power of two in [LECB_MIN_CHUNK, LECB_MAX_CHUNK].
 */
#ifndef LECB_H
#define LECB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LECB_ABI_VERSION 3u
#define LECB_MAX_CODE_LEN 16u
#define LECB_LANE_SYMBOLS 256u   /* a chunk has one lane per 256 symbols ... */
#define LECB_LANES_MAX 16u       /* ... and at most 16 */
#define LECB_MIN_CHUNK 256u
#define LECB_MAX_CHUNK 65536u
#define LECB_CONTAINER_HEADER_BYTES 560u
#define LECB_NOALLOC_SCRATCH_BYTES (16u << 20)

typedef enum {
    LECB_OK = 0,
    LECB_ERR_INVALID_ARG = -1,    /* null/misaligned pointer, bad chunk or max_len */
    LECB_ERR_CAPACITY = -2,       /* output buffer too small (host or device check) */
    LECB_ERR_TOO_LARGE = -3,      /* payload would need >= 2^32 words */
    LECB_ERR_NO_SYMBOLS = -4,     /* histogram empty, or more coded symbols than 2^max_len */
    LECB_ERR_HIP = -5,            /* a HIP runtime call failed */
    LECB_ERR_WORKSPACE = -6,      /* workspace too small */
    LECB_ERR_SCRATCH = -7,        /* input too large for the static scratch of lecb_encode_noalloc */
    LECB_ERR_UNCODED_SYMBOL = -16,/* device: input holds a byte whose code length is 0 */
    LECB_ERR_CORRUPT = -17        /* device: stream is not a valid v3 stream for these arguments */
} lecb_status;

/* Canonical codebook, host side.  Fully determined by len[]. */
typedef struct {
    uint32_t max_len;     /* length limit it was built with (1..16) */
    uint32_t num_coded;   /* symbols with len > 0 */
    uint8_t len[256];     /* code length per byte value; 0 = no code word */
    uint16_t code[256];   /* right-aligned code word; its MSB is the first bit emitted */
} lecb_codebook;

/* Written by the device at the end of a call (read it after synchronising). */
typedef struct {
    uint64_t bytes;        /* encode: stream size in bytes; decode: stream bytes used */
    uint64_t payload_bits; /* exact coded bits = sum over symbols of their code length */
    int32_t status;        /* LECB_OK or a device-detected lecb_status */
    uint32_t reserved;
} lecb_result;

/* ------------------------------------------------------------------ host only, pure */

uint32_t lecb_abi_version(void);
const char* lecb_status_str(int status);

/* ceil(n / chunk); 0 on a bad chunk. */
uint64_t lecb_num_chunks(uint64_t n, uint32_t chunk);
/* Bytes before the payload: align16(4*nc) + align16(2*nc*G). */
uint64_t lecb_header_bytes(uint64_t n, uint32_t chunk);
/* Largest stream any codebook with lengths <= max_len can produce, rounded
 * up to 16 bytes: align16(header + 4 * sum over lanes of ceil(m*max_len/32))
 * for lanes of m symbols -- the size when every symbol has a max_len-bit
 * code word.  0 on bad arguments or n >= 2^60. */
uint64_t lecb_encoded_bound(uint64_t n, uint32_t chunk, uint32_t max_len);
/* Workspace bytes an encode or decode of n symbols with this chunk needs. */
uint64_t lecb_workspace_bytes(uint64_t n, uint32_t chunk);

/* Build a canonical, length-limited optimal codebook from a histogram.
 * Frequencies are first raised to at least min_freq (min_freq = 1 gives every
 * byte value a code word, as a fixed codebook needs; 0 keeps absent symbols
 * uncoded).  Lengths minimise sum(F*len) subject to len <= max_len
 * (package-merge; ties: lower frequency, then lower byte value, merges first;
 * a single coded symbol gets length 1).  Basis: "Single-Stage Huffman Encoder
 * for ML Compression", Methodology steps 2-3; "Lossless Compression for LLM
 * Tensor Incremental Snapshots", Technical framework step 3.
 * Errors: INVALID_ARG (null, max_len not in 1..16), NO_SYMBOLS (all zero, or
 * more than 2^max_len coded symbols). */
int lecb_build_codebook(const uint64_t hist[256], uint32_t max_len, uint32_t min_freq,
                        lecb_codebook* out);

/* Canonical codes for given lengths (decoder side, or a stored container).
 * Errors: INVALID_ARG if a length exceeds 16 or the lengths violate Kraft. */
int lecb_codebook_from_lengths(const uint8_t len[256], lecb_codebook* out);

/* Size accounting of one coded stream ("Single-Stage Huffman Encoder for ML
 * Compression", Key contributions and Results: the fixed codebook is compared
 * with per-shard Huffman coding and with the Shannon bound).  From the data's
 * histogram and the code lengths used:
 *   n             = sum hist;
 *   payload_bits  = sum hist[s] * len[s]       (what any encoder must emit);
 *   shannon_bits  = n * H, H = -sum p log2 p   (empirical entropy, fp64);
 *   optimal_bits  = payload bits of the optimal length-limited code built
 *                   from this histogram itself (no clamp, limit max_len);
 *   uncoded       = number of symbols whose length is 0 (cannot be coded).
 * Errors: INVALID_ARG (null pointer, max_len not in 1..16). */
typedef struct {
    uint64_t n;
    uint64_t payload_bits;
    uint64_t optimal_bits;
    uint64_t uncoded;
    double shannon_bits;
} lecb_stats;
int lecb_stream_stats(const uint64_t hist[256], const uint8_t len[256], uint32_t max_len,
                      lecb_stats* out);

/* Codebook refresh rule for a drifting stream in fixed-codebook mode.  The
 * page ("Single-Stage Huffman Encoder for ML Compression", Limitations and
 * future work, distribution drift) names adaptive refresh as open work; the
 * rule here: the batch (host histogram `hist`) keeps `cur` unless
 *     bits_cur * 10^6 > bits_opt * (10^6 + tol_ppm),
 * with bits_cur = sum f[s]*len_cur[s] (infinite when a byte present in the
 * batch has no code word in `cur`) and bits_opt the same sum for the best
 * fixed codebook of the batch (lecb_build_codebook with min_freq 1 and
 * max_len).  *out = that codebook when refreshing, else a copy of *cur (out
 * may equal cur); *refreshed = 1 / 0; *bits_cur (UINT64_MAX when not
 * codable) and *bits_opt when non-NULL.  Host only, no allocation. */
int lecb_drift_check(const uint64_t hist[256], const lecb_codebook* cur, uint32_t max_len,
                     uint32_t tol_ppm, lecb_codebook* out, int* refreshed, uint64_t* bits_cur,
                     uint64_t* bits_opt);

/* Size of the device-resident codebook (encode table + decode tables). */
uint64_t lecb_device_codebook_bytes(void);

/* Bf16 container header (per-tensor mode stores its two length tables):
 * magic "LECB", u16 version 1, u16 kind 1, u64 n, u32 chunk, u32 max_len,
 * u8 len_hi[256], u8 len_lo[256], u64 bytes_hi, u64 bytes_lo, zero pad to
 * 560 bytes; stream_hi follows, zero-padded to 16 bytes, then stream_lo. */
int lecb_container_write_header(uint8_t out[LECB_CONTAINER_HEADER_BYTES], uint64_t n,
                                uint32_t chunk, uint32_t max_len, const uint8_t len_hi[256],
                                const uint8_t len_lo[256], uint64_t bytes_hi, uint64_t bytes_lo);
int lecb_container_read_header(const uint8_t in[LECB_CONTAINER_HEADER_BYTES], uint64_t* n,
                               uint32_t* chunk, uint32_t* max_len, uint8_t len_hi[256],
                               uint8_t len_lo[256], uint64_t* bytes_hi, uint64_t* bytes_lo);

/* ------------------------------------------------------------------ device, asynchronous */

/* Zero-fill a workspace (a fill kernel, no memset node). */
int lecb_workspace_init(void* d_ws, uint64_t ws_bytes, void* stream);

/* Place a codebook on the device: "stored on each accelerator" ("Single-Stage
 * Huffman Encoder for ML Compression", Methodology step 3).  d_blob holds
 * lecb_device_codebook_bytes() bytes; the tables are built by a kernel from
 * the codebook passed by value, so `cb` may be reused as soon as this returns. */
int lecb_codebook_upload(const lecb_codebook* cb, void* d_blob, void* stream);

/* Byte histogram f[s] = #{i : in[i] == s} as u64[256] ("frequency analysis",
 * "Single-Stage Huffman Encoder for ML Compression", Overview and Methodology
 * step 1).  accumulate = 0 overwrites d_hist, 1 adds to it. */
int lecb_histogram(const uint8_t* d_in, uint64_t n, uint64_t* d_hist, int accumulate,
                   void* stream);
/* Histograms of the high and low byte planes of 16-bit words in one pass
 * ("Lossless Compression for LLM Tensor Incremental Snapshots", Technical
 * framework steps 1-2). */
int lecb_histogram_bf16(const uint16_t* d_in, uint64_t n, uint64_t* d_hist_hi,
                        uint64_t* d_hist_lo, int accumulate, void* stream);

/* Byte grouping: hi[i] = in[i] >> 8, lo[i] = in[i] & 0xFF, and its inverse
 * ("Lossless Compression for LLM Tensor Incremental Snapshots", Technical
 * framework step 1 and the byte-group restore of the reverse path). */
int lecb_split_bf16(const uint16_t* d_in, uint64_t n, uint8_t* d_hi, uint8_t* d_lo,
                    void* stream);
int lecb_merge_bf16(const uint8_t* d_hi, const uint8_t* d_lo, uint64_t n, uint16_t* d_out,
                    void* stream);

/* Encode n bytes with an uploaded codebook into a v3 stream ("Single-Stage
 * Huffman Encoder for ML Compression", Methodology step 4).  out_capacity must
 * be at least lecb_header_bytes(n, chunk); a payload that does not fit sets
 * status CAPACITY (lecb_encoded_bound gives a size that always fits).
 * d_res receives bytes, payload_bits, status. */
int lecb_encode(const uint8_t* d_in, uint64_t n, const void* d_blob, uint32_t chunk,
                uint8_t* d_out, uint64_t out_capacity, lecb_result* d_res, void* d_ws,
                uint64_t ws_bytes, void* stream);

/* Decode a v3 stream of n symbols into d_out[n] (reverse path of "Lossless
 * Compression for LLM Tensor Incremental Snapshots", Technical framework).
 * stream_bytes must be the exact stream size (lecb_result.bytes of the
 * encode).  The buffer must be readable up to align16(stream_bytes) (the
 * decoder fetches whole 16-byte groups; bytes past stream_bytes are ignored).  A size below the header or not a whole
 * number of payload words returns LECB_ERR_CORRUPT at once.  A stream that is not exactly what
 * lecb_encode produces for these arguments sets status CORRUPT (offset table
 * not increasing or past the stream, lane word counts that disagree with
 * their chunk's words or give words to an empty lane, a bit pattern with no
 * code word, a code word past its lane's last word, a lane word that is
 * never needed, non-zero padding). */
int lecb_decode(const uint8_t* d_stream, uint64_t stream_bytes, const void* d_blob,
                uint32_t chunk, uint64_t n, uint8_t* d_out, lecb_result* d_res, void* d_ws,
                uint64_t ws_bytes, void* stream);

/* lecb_decode with the stream's size taken on the device from the result an
 * encode wrote (d_enc_res->bytes), so an encode -> decode chain needs no host
 * synchronisation.  An encoder status other than LECB_OK, or a size that
 * lecb_decode would refuse, gives status CORRUPT in *d_res. */
int lecb_decode_from_result(const uint8_t* d_stream, const lecb_result* d_enc_res,
                            const void* d_blob, uint32_t chunk, uint64_t n, uint8_t* d_out,
                            lecb_result* d_res, void* d_ws, uint64_t ws_bytes, void* stream);

/* lecb_encode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument, no allocation of any kind.  Its workspace is a static
 * device array of LECB_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends; inputs up to
 * lecb_workspace_bytes(n, chunk) <= LECB_NOALLOC_SCRATCH_BYTES fit (about
 * 4 Gi symbols at chunk 4096), larger ones return LECB_ERR_SCRATCH before
 * any work is enqueued.  The stream, d_res and every other rule are those of
 * lecb_encode.  All calls on one GPU share its array: calls that overlap in
 * time on one GPU (different streams or host threads) race and must be
 * serialised by the caller.  Each call clears the part of the array that must
 * start at zero (a fill kernel, no memset) before its encode. */
int lecb_encode_noalloc(const uint8_t* d_in, uint64_t n, const void* d_blob, uint32_t chunk,
                        uint8_t* d_out, uint64_t out_capacity, lecb_result* d_res, void* stream);

/* Encode one byte plane of 16-bit words without materialising it:
 * plane 1 = high bytes (in >> 8), plane 0 = low bytes (in & 0xFF). */
int lecb_encode_plane(const uint16_t* d_in, uint64_t n, int plane, const void* d_blob,
                      uint32_t chunk, uint8_t* d_out, uint64_t out_capacity,
                      lecb_result* d_res, void* d_ws, uint64_t ws_bytes, void* stream);

/* Both byte planes of 16-bit words in ONE pass over d_in, each with its own
 * codebook ("Lossless Compression for LLM Tensor Incremental Snapshots",
 * Technical framework: byte grouping, then Huffman coding of each group;
 * with codebooks built beforehand, as "Single-Stage Huffman Encoder for ML
 * Compression", Methodology step 4).  Stream "hi" codes in >> 8 with d_blob_hi
 * into d_out_hi, stream "lo" codes in & 0xFF with d_blob_lo into d_out_lo;
 * each stream is the same bytes lecb_encode_plane produces.  d_res2: two
 * lecb_result (hi, lo).  d_ws: lecb_workspace_bytes(n, chunk) (one workspace
 * covers both streams). */
int lecb_encode_bf16(const uint16_t* d_in, uint64_t n, const void* d_blob_hi,
                     const void* d_blob_lo, uint32_t chunk, uint8_t* d_out_hi, uint64_t cap_hi,
                     uint8_t* d_out_lo, uint64_t cap_lo, lecb_result* d_res2, void* d_ws,
                     uint64_t ws_bytes, void* stream);

/* Per-tensor bf16 encode, the classic three steps ("Single-Stage Huffman
 * Encoder for ML Compression", Overview) on byte planes ("Lossless
 * Compression for LLM Tensor Incremental Snapshots", Technical framework):
 * one-pass plane histograms -> read back (synchronises `stream` once) ->
 * host codebook per plane (no clamp, length limit max_len) -> upload ->
 * lecb_encode_bf16.  cb_hi / cb_lo (host) receive the codebooks, whose
 * lengths a container stores.  d_hist: 512 u64 of device scratch (high
 * plane histogram in [0, 256), low plane in [256, 512)).
 * d_res2: two lecb_result (hi, lo).  d_blob_hi/lo: device codebooks.
 * d_ws: lecb_workspace_bytes(n, chunk). */
int lecb_encode_bf16_pertensor(const uint16_t* d_in, uint64_t n, uint32_t chunk,
                               uint32_t max_len, uint64_t* d_hist, void* d_blob_hi,
                               void* d_blob_lo, lecb_codebook* cb_hi, lecb_codebook* cb_lo,
                               uint8_t* d_out_hi, uint64_t cap_hi, uint8_t* d_out_lo,
                               uint64_t cap_lo, lecb_result* d_res2, void* d_ws,
                               uint64_t ws_bytes, void* stream);

/* ---- incremental snapshot delta, fused ("Lossless Compression for LLM
 * Tensor Incremental Snapshots", Technical framework: the delta of two
 * consecutive checkpoints is byte-grouped and Huffman-coded; the delta here is
 * the bitwise XOR of the two bf16 tensors, D[i] = W0[i] ^ W1[i]).  These
 * entries read W0 and W1 (or W0 and the streams) directly, so D is never
 * written to memory: the streams are those of the entries above applied to
 * D, and the decode writes W1 = W0 ^ D.  Arguments as for the bf16 entries
 * above, plus d_w0 / d_w1 (n u16 each, 16-byte aligned). */

/* Histograms of the two byte planes of W0 ^ W1. */
int lecb_histogram_bf16_delta(const uint16_t* d_w0, const uint16_t* d_w1, uint64_t n,
                              uint64_t* d_hist_hi, uint64_t* d_hist_lo, int accumulate,
                              void* stream);

/* lecb_encode_bf16 of W0 ^ W1 (both planes in one pass, fixed codebooks). */
int lecb_encode_bf16_delta(const uint16_t* d_w0, const uint16_t* d_w1, uint64_t n,
                           const void* d_blob_hi, const void* d_blob_lo, uint32_t chunk,
                           uint8_t* d_out_hi, uint64_t cap_hi, uint8_t* d_out_lo, uint64_t cap_lo,
                           lecb_result* d_res2, void* d_ws, uint64_t ws_bytes, void* stream);

/* lecb_encode_bf16_pertensor of W0 ^ W1 (per-tensor codebooks of the delta
 * planes; synchronises `stream` once, like lecb_encode_bf16_pertensor). */
int lecb_encode_bf16_delta_pertensor(const uint16_t* d_w0, const uint16_t* d_w1, uint64_t n,
                                     uint32_t chunk, uint32_t max_len, uint64_t* d_hist,
                                     void* d_blob_hi, void* d_blob_lo, lecb_codebook* cb_hi,
                                     lecb_codebook* cb_lo, uint8_t* d_out_hi, uint64_t cap_hi,
                                     uint8_t* d_out_lo, uint64_t cap_lo, lecb_result* d_res2,
                                     void* d_ws, uint64_t ws_bytes, void* stream);

/* Decode both delta planes and write W1 = W0 ^ (hi << 8 | lo) in the same
 * launch (the decoded planes never go to memory).  d_w1 may not be d_w0. */
int lecb_decode_bf16_delta(const uint8_t* d_hi, uint64_t hi_bytes, const uint8_t* d_lo,
                           uint64_t lo_bytes, const void* d_blob_hi, const void* d_blob_lo,
                           uint32_t chunk, uint64_t n, const uint16_t* d_w0, uint16_t* d_w1,
                           lecb_result* d_res2, void* d_ws, uint64_t ws_bytes, void* stream);

/* As lecb_decode_bf16_delta, with the stream sizes read on the device from
 * the encoder's two results (d_enc_res2), so encode -> decode needs no host
 * synchronisation. */
int lecb_decode_bf16_delta_from_results(const uint8_t* d_hi, const uint8_t* d_lo,
                                        const lecb_result* d_enc_res2, const void* d_blob_hi,
                                        const void* d_blob_lo, uint32_t chunk, uint64_t n,
                                        const uint16_t* d_w0, uint16_t* d_w1,
                                        lecb_result* d_res2, void* d_ws, uint64_t ws_bytes,
                                        void* stream);

/* Fixed-codebook encode of one batch of a drifting stream with the refresh
 * rule of lecb_drift_check: histogram of the batch (device) -> read back
 * (synchronises `stream` once; a 4 KiB pinned host buffer per host thread,
 * allocated on first use) -> lecb_drift_check(tol_ppm) -> on refresh the new
 * codebook is built on the host and uploaded into d_blob -> lecb_encode.
 * cb (host) in: the codebook d_blob holds; out: the one this batch was coded
 * with.  *refreshed = 1 when it changed.  d_hist: 256 u64 of device scratch.
 * The stream decodes with lecb_decode and the codebook in *cb. */
int lecb_encode_adaptive(const uint8_t* d_in, uint64_t n, uint32_t chunk, uint32_t max_len,
                         uint32_t tol_ppm, uint64_t* d_hist, lecb_codebook* cb, void* d_blob,
                         int* refreshed, uint8_t* d_out, uint64_t cap, lecb_result* d_res,
                         void* d_ws, uint64_t ws_bytes, void* stream);

/* Decode both byte planes in ONE launch (the two streams' decode units run
 * side by side) into d_out_hi[n] and d_out_lo[n]; same rules as lecb_decode
 * for each stream.  d_res2: two lecb_result (hi, lo).  d_ws:
 * lecb_workspace_bytes(n, chunk).  Reverse path of "Lossless Compression for
 * LLM Tensor Incremental Snapshots", Technical framework (Huffman-decode of
 * each byte group). */
int lecb_decode_bf16_planes(const uint8_t* d_hi, uint64_t hi_bytes, const uint8_t* d_lo,
                            uint64_t lo_bytes, const void* d_blob_hi, const void* d_blob_lo,
                            uint32_t chunk, uint64_t n, uint8_t* d_out_hi, uint8_t* d_out_lo,
                            lecb_result* d_res2, void* d_ws, uint64_t ws_bytes, void* stream);

/* lecb_decode_bf16_planes with both streams' sizes taken on the device from
 * the two results an encode wrote (d_enc_res2, hi then lo): the two byte
 * planes, not merged.  Errors as lecb_decode_from_result. */
int lecb_decode_bf16_planes_from_results(const uint8_t* d_hi, const uint8_t* d_lo,
                                         const lecb_result* d_enc_res2, const void* d_blob_hi,
                                         const void* d_blob_lo, uint32_t chunk, uint64_t n,
                                         uint8_t* d_out_hi, uint8_t* d_out_lo, lecb_result* d_res2,
                                         void* d_ws, uint64_t ws_bytes, void* stream);

/* lecb_decode_bf16 with both streams' sizes taken on the device from the
 * two results an encode wrote (d_enc_res2, hi then lo), so a per-tensor
 * encode -> decode chain needs no host synchronisation; errors as in
 * lecb_decode_from_result. */
int lecb_decode_bf16_from_results(const uint8_t* d_hi, const uint8_t* d_lo,
                                  const lecb_result* d_enc_res2, const void* d_blob_hi,
                                  const void* d_blob_lo, uint32_t chunk, uint64_t n,
                                  uint16_t* d_out, lecb_result* d_res2,
                                  void* d_ws, uint64_t ws_bytes, void* stream);

/* Decode both planes and restore the 16-bit words, out[i] = hi[i] << 8 | lo[i]:
 * the reverse path of "Lossless Compression for LLM Tensor Incremental
 * Snapshots", Technical framework (Huffman-decode each byte group, then
 * restore the byte groups), in ONE launch: the lanes that decode the two
 * planes of the same 256 elements sit side by side and write the restored
 * words directly (the planes never go to memory).  d_out: n u16, 16-byte
 * aligned.  d_ws: lecb_workspace_bytes(n, chunk).  Errors as lecb_decode,
 * per plane. */
int lecb_decode_bf16(const uint8_t* d_hi, uint64_t hi_bytes, const uint8_t* d_lo,
                     uint64_t lo_bytes, const void* d_blob_hi, const void* d_blob_lo,
                     uint32_t chunk, uint64_t n, uint16_t* d_out,
                     lecb_result* d_res2, void* d_ws, uint64_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ codebooks built on the device
 * Per-shard codebook generation ("Single-Stage Huffman Encoder for ML
 * Compression", Overview: frequency analysis, codebook generation, codebook
 * transmission) done on the accelerator, so a per-tensor encode needs no host
 * round trip.  The result is bit for bit the one of lecb_build_codebook with
 * the same arguments (package-merge, the same tie rule, canonical codes), in
 * the device layout of lecb_codebook_upload. */

/* For p < nplanes (1..4): the codebook of histogram d_hist[256*p : 256*p+256]
 * (u64 counts in device memory), frequencies raised to min_freq, lengths at
 * most max_len (1..16), written to the device codebook d_blob[p] (host array
 * of device pointers, each lecb_device_codebook_bytes() bytes).  When no code
 * exists (every count 0 after the clamp, or more than 2^max_len coded
 * values) the device codebook holds no code word, and an encode with it
 * reports LECB_ERR_UNCODED_SYMBOL.  Two launches on `stream`; no
 * synchronisation. */
int lecb_build_codebook_device(const uint64_t* d_hist, uint32_t nplanes, uint32_t max_len,
                               uint32_t min_freq, void* const d_blob[], void* stream);

/* The host codebook (lengths and canonical codes) of a device codebook, e.g.
 * for the container header.  Copies 1 KiB and synchronises `stream`. */
int lecb_codebook_download(const void* d_blob, lecb_codebook* out, void* stream);

/* The codebook half of a per-tensor encode, built on the host: plane
 * histograms of the n elements of d_in (elem_bytes 2: bf16 planes, high byte
 * first; 4: fp32 planes, byte 3 first) into d_hist (u64[256*elem_bytes]) ->
 * read back (synchronises `stream` once) -> one optimal codebook per plane
 * (min_freq 0) returned in cb[] and uploaded to d_blob[] (host array of
 * device pointers).  lecb_encode_bf16 / lecb_encode_fp32 with these blobs
 * then give the streams of lecb_encode_bf16_pertensor / _fp32_pertensor.
 * n must be > 0. */
int lecb_pertensor_codebooks(const void* d_in, uint32_t elem_bytes, uint64_t n, uint32_t max_len,
                             uint64_t* d_hist, void* const d_blob[], lecb_codebook cb[], void* stream);

/* Per-tensor encodes whose codebooks are built on the device: plane
 * histograms -> lecb_build_codebook_device (min_freq 0) -> the two-plane /
 * four-plane encode.  Same streams as the _pertensor entries; they neither
 * synchronise nor return host codebooks (lecb_codebook_download gives them). */
int lecb_encode_bf16_pertensor_nosync(const uint16_t* d_in, uint64_t n, uint32_t chunk,
                                      uint32_t max_len, uint64_t* d_hist, void* d_blob_hi,
                                      void* d_blob_lo, uint8_t* d_out_hi, uint64_t cap_hi,
                                      uint8_t* d_out_lo, uint64_t cap_lo, lecb_result* d_res2,
                                      void* d_ws, uint64_t ws_bytes, void* stream);
int lecb_encode_bf16_delta_pertensor_nosync(const uint16_t* d_w0, const uint16_t* d_w1, uint64_t n,
                                            uint32_t chunk, uint32_t max_len, uint64_t* d_hist,
                                            void* d_blob_hi, void* d_blob_lo, uint8_t* d_out_hi,
                                            uint64_t cap_hi, uint8_t* d_out_lo, uint64_t cap_lo,
                                            lecb_result* d_res2, void* d_ws, uint64_t ws_bytes,
                                            void* stream);

/* ------------------------------------------------------------------ 32-bit elements (fp32)
 * Byte grouping with four planes ("Lossless Compression for LLM Tensor
 * Incremental Snapshots", Technical framework step 1 and Key design item 1,
 * the byte-group size): plane p holds byte 3-p of every element (elements
 * little-endian), so plane 0 = sign and high exponent bits, plane 3 = the
 * lowest mantissa byte.  Every per-plane array below (codebooks, streams,
 * capacities, results, histograms) is in that plane order.  Works on any
 * 32-bit elements; n counts elements.  The workspace is the one of
 * lecb_workspace_bytes(n, chunk): the two halves of the work use it one
 * after the other on `stream`. */

/* Histograms of the four planes: d_hist = u64[4*256], plane p at 256*p.
 * accumulate != 0 adds to d_hist instead of overwriting it. */
int lecb_histogram_fp32(const uint32_t* d_in, uint64_t n, uint64_t* d_hist, int accumulate,
                        void* stream);

/* out[i] = planes[0][i] << 24 | planes[1][i] << 16 | planes[2][i] << 8 | planes[3][i].
 * d_planes: host array of four device pointers. */
int lecb_merge_fp32(const uint8_t* const d_planes[4], uint64_t n, uint32_t* d_out, void* stream);

/* Encode the four planes with four device codebooks (host arrays of device
 * pointers d_blob, d_out and of capacities cap); d_res4 = four results.  Two
 * launch pairs, each coding two planes in one pass over the elements.
 * Errors as lecb_encode_bf16, per plane. */
int lecb_encode_fp32(const uint32_t* d_in, uint64_t n, const void* const d_blob[4], uint32_t chunk,
                     uint8_t* const d_out[4], const uint64_t cap[4], lecb_result* d_res4, void* d_ws,
                     uint64_t ws_bytes, void* stream);

/* Per-tensor mode: plane histograms (d_hist, u64[1024]) -> read back -> four
 * optimal codebooks built on the host (returned in cb[4], absent bytes get
 * no code) -> uploaded to d_blob[4] -> lecb_encode_fp32.  Synchronises
 * `stream` once (the histogram read-back). */
int lecb_encode_fp32_pertensor(const uint32_t* d_in, uint64_t n, uint32_t chunk, uint32_t max_len,
                               uint64_t* d_hist, void* const d_blob[4], lecb_codebook cb[4],
                               uint8_t* const d_out[4], const uint64_t cap[4], lecb_result* d_res4,
                               void* d_ws, uint64_t ws_bytes, void* stream);

/* lecb_encode_fp32_pertensor with the four codebooks built on the device
 * (see lecb_build_codebook_device): never synchronises. */
int lecb_encode_fp32_pertensor_nosync(const uint32_t* d_in, uint64_t n, uint32_t chunk,
                                      uint32_t max_len, uint64_t* d_hist, void* const d_blob[4],
                                      uint8_t* const d_out[4], const uint64_t cap[4],
                                      lecb_result* d_res4, void* d_ws, uint64_t ws_bytes,
                                      void* stream);

/* Decode the four streams (exact sizes in stream_bytes[4]) and restore the
 * 32-bit elements in ONE launch (the four lanes of the same 256 elements sit
 * side by side and write the elements directly).  Errors as lecb_decode_bf16. */
int lecb_decode_fp32(const uint8_t* const d_stream[4], const uint64_t stream_bytes[4],
                     const void* const d_blob[4], uint32_t chunk, uint64_t n, uint32_t* d_out,
                     lecb_result* d_res4, void* d_ws, uint64_t ws_bytes, void* stream);

/* lecb_decode_fp32 with the four sizes read on the device from the results
 * an encode wrote (d_enc_res4), so encode -> decode needs no host
 * synchronisation. */
int lecb_decode_fp32_from_results(const uint8_t* const d_stream[4], const lecb_result* d_enc_res4,
                                  const void* const d_blob[4], uint32_t chunk, uint64_t n,
                                  uint32_t* d_out, lecb_result* d_res4,
                                  void* d_ws, uint64_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LECB_H */
