// Internal declarations shared by the host runtime and the HIP kernels.
#pragma once

#include <cstddef>
#include <cstdint>

#include "lecb.h"

namespace lecb {

// ---------------------------------------------------------------- device codebook
// Decode table `dec`, one probe per code word.  With v the next 16 bits
// (left-aligned window) and long_base = the left-aligned end of the code
// words of at most LUT_BITS bits (a multiple of 16, so the windows below it
// are exactly the code words of at most LUT_BITS bits):
//   * dec[i], i < long_base / 16: the code word that the LUT_BITS-bit prefix i
//     starts with;
//   * dec[long_base / 16 + (v - long_base)], v >= long_base: the longer code
//     word window v starts with (a complete code has at most 256 of them, each
//     covering at most 2^(16-13) windows: LONG_SIZE entries);
// so the entry of v is dec[med3(v >> 4, v - long_sub, DEC_SIZE)] with
// long_sub = long_base - long_base / 16 (the first index wins below
// long_base, the second from it on).  Entries are (sym << 8) | len; a window
// that starts no code word (an incomplete code), the entries past the long
// windows and the sentinel dec[DEC_SIZE] are DEC_INVALID: length 16 with
// bit 7 set.
constexpr int LUT_BITS = 12;
constexpr int LUT_SIZE = 1 << LUT_BITS;
constexpr int LONG_SIZE = 2048;
constexpr int DEC_SIZE = LUT_SIZE + LONG_SIZE;
constexpr int DEC_ENTRIES = DEC_SIZE + 8;   // the sentinel, then padding to 16 bytes
constexpr uint16_t DEC_INVALID = 0x0090;

struct DeviceCodebook {
    uint32_t enc[256];           // (code << 5) | len ; len 0 = byte has no code word
    uint16_t dec[DEC_ENTRIES];   // decode table (above)
    uint32_t limit[17];          // per length l: (first[l] + count[l]) << (16 - l), non-decreasing in l
    uint32_t first[17];          // first canonical code of length l
    uint32_t base[17];           // index in `sorted` of the first symbol of length l
    uint8_t sorted[256];         // coded symbols by (length, byte value)
    uint32_t max_len;
    uint32_t num_coded;
    uint32_t long_base;          // limit[LUT_BITS]
    uint32_t long_sub;           // long_base - long_base / 16
    uint32_t pad[1];
};
static_assert(sizeof(DeviceCodebook) % 16 == 0, "device codebook must stay 16-byte sized");
static_assert(offsetof(DeviceCodebook, dec) % 16 == 0, "the decode table is copied in 16-byte pieces");

// Everything the upload kernel needs, passed by value as a kernel argument.
struct CodebookArgs {
    uint32_t enc[256];
    uint32_t first[17];
    uint32_t count[17];
    uint32_t base[17];
    uint8_t sorted[256];
    uint32_t max_len;
    uint32_t num_coded;
};

// ---------------------------------------------------------------- workspace
// Encode: exit counter and accumulators, followed by the payload words of
// each count range (written by the count launch, turned into first words by
// the offsets launch, read by the pack launch of the same call).  Decode:
// exit counter + status.  A workspace holds two of them (header + one u64
// per chunk and four more each, 256-byte aligned; there are never more
// ranges than chunks + 3): a two-stream encode uses both; everything else
// uses the first.
// Two more headers follow, for the third and fourth stream of a four-plane
// decode.  The last wave of every call resets the headers, so only the first
// use needs a zero-filled workspace.
struct WsHeader {
    uint32_t unused0;
    uint32_t exit_count;
    uint32_t unused1;
    int32_t status;
    uint64_t bits;
    uint64_t words;
    uint64_t pad[4];
};
static_assert(sizeof(WsHeader) == 64, "workspace header is 64 bytes");

inline uint64_t align16(uint64_t x) { return (x + 15) & ~uint64_t(15); }
inline int ilog2(uint32_t x) {
    int l = 0;
    while ((1u << l) < x) ++l;
    return l;
}
inline bool valid_chunk(uint32_t chunk) {
    return chunk >= LECB_MIN_CHUNK && chunk <= LECB_MAX_CHUNK && (chunk & (chunk - 1)) == 0;
}
// Lanes per chunk: one per 256 symbols, at most 16 (a valid chunk has at least 256 symbols).
inline uint32_t lanes_per_chunk(uint32_t chunk) {
    return chunk / LECB_LANE_SYMBOLS < LECB_LANES_MAX ? chunk / LECB_LANE_SYMBOLS : LECB_LANES_MAX;
}
inline uint64_t table_bytes(uint64_t nc) { return align16(4 * nc); }
// The u16 word count of every lane (G per chunk), padded to 16 bytes.
inline uint64_t count_bytes(uint64_t nc, uint32_t chunk) { return align16(2 * nc * lanes_per_chunk(chunk)); }
// Bytes of one stream's part of the workspace: header + one u64 per chunk and four more.
inline uint64_t ws_stream_bytes(uint64_t nc) { return (sizeof(WsHeader) + 8 * (nc + 4) + 255) & ~uint64_t(255); }
// Two more headers after the stream parts (the four streams of a four-plane decode).
constexpr uint64_t WS_EXTRA_BYTES = 256;
inline uint64_t ws_total_bytes(uint64_t nc) { return 2 * ws_stream_bytes(nc) + WS_EXTRA_BYTES; }
// ceil(n / chunk) without the wrap of n + chunk - 1 near 2^64; 0 on a bad chunk.
inline uint64_t num_chunks_of(uint64_t n, uint32_t chunk) {
    return valid_chunk(chunk) ? n / chunk + (n % chunk != 0) : 0;
}
// Stream bytes before the payload (chunk table, lane word counts); 0 on a bad chunk.
inline uint64_t header_bytes_of(uint64_t n, uint32_t chunk) {
    const uint64_t nc = num_chunks_of(n, chunk);
    return nc ? table_bytes(nc) + count_bytes(nc, chunk) : 0;
}
inline uint64_t ws_bytes_of(uint64_t n, uint32_t chunk) { return ws_total_bytes(num_chunks_of(n, chunk)); }
// Offset of stream k's header (k < 4): the two stream parts, then the extra headers.
inline uint64_t ws_header_offset(int k, uint64_t nc) {
    return k < 2 ? k * ws_stream_bytes(nc) : 2 * ws_stream_bytes(nc) + (k - 2) * sizeof(WsHeader);
}

// ---------------------------------------------------------------- host helpers
int build_lengths(const uint64_t freq[256], uint32_t max_len, uint32_t min_freq,
                  uint8_t len_out[256]);
int canonical_from_lengths(const uint8_t len[256], lecb_codebook* out);

// ---------------------------------------------------------------- launches (kernels_*.hip)
// Input kinds of the encode kernel.  ENC_PAIR codes both bytes of 16-bit
// words in one pass: stream 0 = high bytes, stream 1 = low bytes.
// ENC_PAIR_XOR: both planes of w0[i] ^ w1[i] (the incremental snapshot delta)
// ENC_PAIR32_HI / ENC_PAIR32_LO: the two bytes of the upper / lower 16 bits of
// 32-bit elements (bytes 3 and 2 / bytes 1 and 0), as two streams.
enum EncodeMode {
    ENC_BYTES = 0,
    ENC_PLANE_LO = 1,
    ENC_PLANE_HI = 2,
    ENC_PAIR = 3,
    ENC_PAIR_XOR = 4,
    ENC_PAIR32_HI = 5,
    ENC_PAIR32_LO = 6,
    ENC_NUM_MODES = 7
};
// Modes that write two streams (st[0] and st[1]).
constexpr bool two_stream_mode(int m) {
    return m == ENC_PAIR || m == ENC_PAIR_XOR || m == ENC_PAIR32_HI || m == ENC_PAIR32_LO;
}

struct EncodeStream {
    const DeviceCodebook* cb;
    uint8_t* out;            // stream base
    uint64_t capacity;       // bytes
    lecb_result* res;
    WsHeader* ws;            // followed by one u64 per chunk (word totals of the count ranges)
};

struct EncodeLaunch {
    const void* in;          // u8 symbols (ENC_BYTES), u16 words or u32 elements (ENC_PAIR32_*)
    const void* in2;         // ENC_PAIR_XOR: the second u16 tensor (symbols of in ^ in2)
    int mode;                // EncodeMode
    uint64_t n;
    uint32_t chunk;
    uint64_t nc;
    EncodeStream st[2];      // st[1] only for the two-stream modes
};
int launch_encode(const EncodeLaunch& a, void* stream);

// What a decode writes: each stream's bytes to its own output (one or two
// streams), or the byte planes of the same elements restored on the way out
// -- 16-bit words from two streams (high plane first), optionally XORed with
// a second tensor (the snapshot delta), or 32-bit elements from four streams
// (plane p = byte 3 - p).
enum DecodeOut { DEC_OUT_PLANES = 0, DEC_OUT_U16 = 1, DEC_OUT_U16_XOR = 2, DEC_OUT_U32 = 3 };

// Streams of the same n and chunk decoded in one launch; stream k uses
// workspace header ws[k].
struct DecodeLaunch {
    int nstreams;
    int out_kind;                   // DecodeOut
    const lecb_result* dev_sizes;   // non-null: stream sizes are read on the device from these
    const uint8_t* stream_base[4];
    uint64_t stream_bytes[4];
    const DeviceCodebook* cb[4];
    uint8_t* out[4];                // DEC_OUT_PLANES
    uint8_t* merged;                // the restored elements (other kinds)
    const uint8_t* w0;              // DEC_OUT_U16_XOR: element i of the output is w0[i] ^ restored[i]
    lecb_result* res[4];
    WsHeader* ws[4];
    uint32_t chunk;
    uint64_t n;
    uint64_t nc;
};
int launch_decode(const DecodeLaunch& a, void* stream);

int launch_histogram_u8(const uint8_t* in, uint64_t n, uint64_t* hist, int accumulate,
                        void* stream);
int launch_histogram_u16(const uint16_t* in, const uint16_t* in2, uint64_t n, uint64_t* hist_hi,
                         uint64_t* hist_lo, int accumulate, void* stream);
int launch_split(const uint16_t* in, uint64_t n, uint8_t* hi, uint8_t* lo, void* stream);
int launch_merge(const uint8_t* hi, const uint8_t* lo, const uint16_t* w0, uint64_t n, uint16_t* out,
                 void* stream);
// Byte planes of 32-bit elements: hist[0:256] = byte 3, ..., hist[768:1024] = byte 0.
int launch_histogram_u32(const uint32_t* in, uint64_t n, uint64_t* hist, int accumulate, void* stream);
// out[i] = p3[i] << 24 | p2[i] << 16 | p1[i] << 8 | p0[i]
int launch_merge4(const uint8_t* p3, const uint8_t* p2, const uint8_t* p1, const uint8_t* p0, uint64_t n,
                  uint32_t* out, void* stream);
int launch_codebook_upload(const CodebookArgs& args, DeviceCodebook* blob, void* stream);
// Codebooks built on the device from n (1..4) device histograms of 256 u64.
int launch_build_codebooks(const uint64_t* const* hist, DeviceCodebook* const* cb, int n, uint32_t max_len,
                           uint32_t min_freq, void* stream);
int launch_fill_zero(void* ptr, uint64_t bytes, void* stream);
int launch_result(lecb_result* r, uint64_t bytes, uint64_t bits, int32_t status, void* stream);

// Devices the per-device caches of the host code cover (ordinals 0..MAX_DEVICES-1).
constexpr int MAX_DEVICES = 64;
int device_cu_count();

}  // namespace lecb
