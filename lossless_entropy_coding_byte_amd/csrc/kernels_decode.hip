// Huffman decode of stream format v3 back to bytes, and back to 16-bit or
// 32-bit elements when the byte planes are decoded together.
//
// Reverse path of "Lossless Compression for LLM Tensor Incremental
// Snapshots", Technical framework (read, Huffman-decode, restore the byte
// groups); the independent parallel tasks of its Key design item 3 are the
// lanes of the format.
//
// One hardware lane runs one lane of the format (lane geometry: lanes.hpp);
// a wave decodes one task at a time, 4 rows of 16 lanes (the grid is as many
// workgroups as the CUs hold, each looping over its tasks):
//   * P = 1, OUT_PLANES: the rows hold lanes of one stream, one byte per
//     symbol written to that stream's output (a stream's tasks run in
//     workgroups of their own);
//   * P = 2, OUT_U16 / OUT_U16_XOR: rows 2g and 2g + 1 decode the high and the
//     low plane of the same chunks; after every block of 16 symbols lanes L
//     and L ^ 16 swap half of their bytes and each stores 8 restored 16-bit
//     words (16 bytes), XORed with the other snapshot for a delta;
//   * P = 4, OUT_U32: rows 0..3 decode planes 0..3 (bytes 3..0 of the 32-bit
//     elements) of the same chunks; after every block the four lanes i,
//     16 + i, 32 + i, 48 + i transpose their words and each stores 4 restored
//     elements.
// The lanes of a row write neighbouring blocks: a row's block stores cover
// 256 contiguous bytes of output per plane.
//
// Reading: the G lanes of a chunk consume one sequential word stream, the
// chunk's payload, in the format's read order.  Each group keeps a ring of
// 16G payload words in LDS, filled by group-wide loads of consecutive words
// (16 bytes per lane, 4G words per load); before every pair of symbols the
// lanes whose first window word is used up take the next words of the ring,
// in lane order (a count over the group's lanes gives each its word).  The
// ring is topped up every 4 pairs: the load issued at one top-up is written
// to the ring two top-ups later, and a load is issued only when the ring has
// room for it; 4 pairs read at most 4G words, so every word read is in the
// ring.
//
// Bit reader: a 64-bit buffer of the lane's next bits; before every pair,
// when it holds 32 bits or fewer (the format's "first window word used up"),
// the next word comes in below them, so it holds more than 32 bits, enough
// for two code words of at most 16 bits.  Every code word is one lookup in
// the decode table (LDS; for two and four planes the longer code words are
// read from the codebook in memory).  Every structural rule of the format is
// checked; a violation sets status CORRUPT.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "lanes.hpp"

namespace lecb {

namespace {

constexpr uint32_t ROW_WORDS = 256;   // ring words per row of 16 lanes (16 per lane)
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

struct DecStream {
    const uint32_t* table;
    const uint16_t* nw;
    const uint32_t* payload;
    uint64_t payload_words;   // words present in the caller's buffer
    const DeviceCodebook* cb;
    uint64_t header_bytes;
    uint64_t table_pad_from, table_pad_to;   // stream bytes that must be zero
    uint64_t nw_pad_from, nw_pad_to;
    const uint8_t* stream;
    uint8_t* out;             // OUT_PLANES: the decoded bytes of this stream
    lecb_result* res;
    WsHeader* ws;
};

struct DecArgs {
    const lecb_result* sizes;  // non-null: stream k's size is sizes[k].bytes (an encoder's result)
    uint32_t chunk;
    uint64_t n;
    uint64_t nc;
    uint32_t wg_per_group;     // workgroup tasks (NW tasks each) of one stream (OUT_PLANES) or of the call
    uint32_t wg_stride;        // workgroups launched per stream (OUT_PLANES) or in all; each loops over
                               // its workgroup tasks bid, bid + wg_stride, ...  (stream = blockIdx.x / wg_stride)
    uint32_t nstreams;
    uint8_t* merged;           // OUT_U16, OUT_U16_XOR, OUT_U32: the restored elements
    const uint8_t* w0;         // OUT_U16_XOR: the other snapshot (element i ^ restored i is written)
    DecStream st[4];
};

// One stream per workgroup: its whole decode table.
template <int NW>
struct SharedOne {
    uint32_t ring[NW][4][ROW_WORDS];   // first: every row's ring is 1 KiB-aligned
    uint16_t dec[DEC_ENTRIES];
    unsigned long long bsum[1];        // payload bits of the lanes decoded without fault
    uint32_t flag[1];                  // bit 0: a fault was found
};
// P streams in every workgroup: every stream's whole decode table.  (A
// table entry read from memory instead would make every lookup wait for the
// ring loads in flight: loads complete in order.)  With P = 2 and 12 waves
// this is 72 KiB, with P = 4 and 6 waves 72 KiB: two workgroups per CU.
template <int NW, int P>
struct SharedMany {
    uint32_t ring[NW][4][ROW_WORDS];
    uint16_t dec[P][DEC_ENTRIES];
    unsigned long long bsum[P];
    uint32_t flag[P];
};
template <int NW, int P>
using Shared = std::conditional_t<P == 1, SharedOne<NW>, SharedMany<NW, P>>;

// What a lane needs of its stream (selected per lane when a wave holds several streams).
struct Lane {
    const uint32_t* table;
    const uint16_t* nw;
    const uint32_t* payload;
    uint64_t payload_words;
    const DeviceCodebook* cb;
    uint8_t* out;
    const uint8_t* stream;
    uint64_t table_pad_from, table_pad_to, nw_pad_from, nw_pad_to;
};

template <int P>
__device__ inline Lane lane_stream(const DecArgs& a, uint32_t k, uint64_t payload_words) {
    Lane l;
#define LECB_PICK(field)                                                              \
    if constexpr (P == 1) {                                                           \
        l.field = a.st[k].field;                                                      \
    } else if constexpr (P == 2) {                                                    \
        l.field = k ? a.st[1].field : a.st[0].field;                                  \
    } else {                                                                          \
        l.field = k & 2 ? (k & 1 ? a.st[3].field : a.st[2].field)                     \
                        : (k & 1 ? a.st[1].field : a.st[0].field);                    \
    }
    LECB_PICK(table)
    LECB_PICK(nw)
    LECB_PICK(payload)
    LECB_PICK(cb)
    LECB_PICK(out)
    LECB_PICK(stream)
    LECB_PICK(table_pad_from)
    LECB_PICK(table_pad_to)
    LECB_PICK(nw_pad_from)
    LECB_PICK(nw_pad_to)
#undef LECB_PICK
    l.payload_words = payload_words;
    return l;
}

// Index of the decode-table entry of the code word that the next bits `top`
// (MSB first) start with: the first LUT_BITS bits below long_base, the window
// offset past it, the sentinel beyond the table (see DeviceCodebook::dec).
__device__ inline uint32_t dec_index(uint32_t top, uint32_t long_sub) {
    const int a = (int)(top >> (32 - LUT_BITS));
    const int b = (int)(top >> 16) - (int)long_sub;
    int r;   // median of (a, b, DEC_SIZE) = min(max(a, b), DEC_SIZE), as a <= DEC_SIZE
    asm("v_med3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(DEC_SIZE));
    return (uint32_t)r;
}

// The symbols (byte 1) of four table entries as one little-endian word.
__device__ inline uint32_t syms4(const uint32_t (&e)[4]) {
    const uint32_t p01 = __builtin_amdgcn_perm(e[1], e[0], 0x0c0c0501u);
    const uint32_t p23 = __builtin_amdgcn_perm(e[3], e[2], 0x0c0c0501u);
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}

// 16 restored 16-bit words from the high-plane bytes of 16 symbols (lane L of
// an even row, w[0..3]) and the low-plane bytes (lane L ^ 16, odd row): the
// pair swaps half of its words, then the high lane builds words 0..7 and the
// low lane words 8..15 (little-endian: low byte first).
__device__ inline v4u restore_u16(const uint32_t (&w)[4], uint32_t odd) {
    const uint32_t s0 = __shfl_xor(odd ? w[0] : w[2], 16, 64);
    const uint32_t s1 = __shfl_xor(odd ? w[1] : w[3], 16, 64);
    const uint32_t h0 = odd ? s0 : w[0], h1 = odd ? s1 : w[1];
    const uint32_t l0 = odd ? w[2] : s0, l1 = odd ? w[3] : s1;
    v4u o;
    o.x = __builtin_amdgcn_perm(h0, l0, 0x05010400u);
    o.y = __builtin_amdgcn_perm(h0, l0, 0x07030602u);
    o.z = __builtin_amdgcn_perm(h1, l1, 0x05010400u);
    o.w = __builtin_amdgcn_perm(h1, l1, 0x07030602u);
    return o;
}

// 16 restored 32-bit elements from the four rows q = 0..3 holding the bytes of
// planes 0..3 (element bytes 3..0) of the same 16 symbols: the lane of row q
// gathers word q of every plane (three exchanges) and builds elements
// 4q..4q+3.
__device__ inline v4u restore_u32(const uint32_t (&w)[4], uint32_t q) {
    uint32_t x0 = 0, x1 = 0, x2 = 0, x3 = 0;  // word q of planes 0..3
    const uint32_t i = threadIdx.x & 15u;
#pragma unroll
    for (uint32_t r = 0; r < 4; ++r) {
        // round r: row q reads row (q + r) & 3, which sends its word (row - r) & 3
        const uint32_t src = (q + r) & 3u;
        const uint32_t want = (q - r) & 3u;
        // (masks rather than an index: the words stay in registers)
        const uint32_t mine = (w[0] & (0u - (uint32_t)(want == 0))) | (w[1] & (0u - (uint32_t)(want == 1))) |
                              (w[2] & (0u - (uint32_t)(want == 2))) | (w[3] & (0u - (uint32_t)(want == 3)));
        const uint32_t got = r ? __shfl(mine, (int)((src << 4) | i), 64) : mine;
        x0 = src == 0 ? got : x0;
        x1 = src == 1 ? got : x1;
        x2 = src == 2 ? got : x2;
        x3 = src == 3 ? got : x3;
    }
    // element k: bytes [x3[k], x2[k], x1[k], x0[k]] (little-endian)
    const uint32_t a01 = __builtin_amdgcn_perm(x0, x1, 0x05010400u);
    const uint32_t b01 = __builtin_amdgcn_perm(x0, x1, 0x07030602u);
    const uint32_t a23 = __builtin_amdgcn_perm(x2, x3, 0x05010400u);
    const uint32_t b23 = __builtin_amdgcn_perm(x2, x3, 0x07030602u);
    v4u o;
    o.x = __builtin_amdgcn_perm(a01, a23, 0x05040100u);
    o.y = __builtin_amdgcn_perm(a01, a23, 0x07060302u);
    o.z = __builtin_amdgcn_perm(b01, b23, 0x05040100u);
    o.w = __builtin_amdgcn_perm(b01, b23, 0x07060302u);
    return o;
}

// The lane's index in its wave, from an asm statement that the compiler
// cannot move or merge: a value derived from it is computed where it is used
// instead of being kept in a register through a loop.
__device__ inline uint32_t lane_index_fresh() {
    uint32_t lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    return lane;
}

// Waves per SIMD the register budget is sized for: two workgroups of the
// largest size per CU (16 waves: 8 per SIMD, 64 VGPRs; 12 waves: 6 per SIMD,
// 85 VGPRs; 6 waves: 3 per SIMD), or one 16-wave workgroup of two or four
// planes (4 per SIMD, 128 VGPRs).  No variant may spill registers (the build
// rejects scratch use).
template <int NT>
constexpr int decode_waves_per_simd(int p) { return NT == 768 ? 6 : NT == 384 ? 3 : (NT == 1024 && p > 1) ? 4 : 8; }

template <int NT, int P, int OUT, int LG>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<NT>(P), 8))) void decode_kernel(DecArgs a) {
    static_assert(P == 1 || OUT != DEC_OUT_PLANES, "plane outputs decode one stream per workgroup");
    constexpr int NW = NT / 64;
    constexpr uint32_t G = 1u << LG;
    constexpr uint32_t R = 16 * G;                    // ring words of a group
    __shared__ __attribute__((aligned(16))) Shared<NW, P> S;
    const int tid = threadIdx.x;
    constexpr uint32_t CPT = (4 / P) * (16u >> LG);
    constexpr int NS = P == 1 ? 1 : P;  // streams in this workgroup
    // P == 1: the workgroup's stream and its first workgroup task
    const uint32_t sidx = P == 1 ? blockIdx.x / a.wg_stride : 0u;
    const uint32_t bid0 = P == 1 ? blockIdx.x - sidx * a.wg_stride : blockIdx.x;

    // ---- tables
    if constexpr (P == 1) {
        const v4u* src = reinterpret_cast<const v4u*>(a.st[sidx].cb->dec);
        v4u* dst = reinterpret_cast<v4u*>(S.dec);
        for (int x = tid; x < DEC_ENTRIES * 2 / 16; x += NT) dst[x] = src[x];
    } else {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const v4u* src = reinterpret_cast<const v4u*>(a.st[q].cb->dec);
            v4u* dst = reinterpret_cast<v4u*>(&S.dec[q][0]);
            for (int x = tid; x < DEC_ENTRIES * 2 / 16; x += NT) dst[x] = src[x];
        }
    }
    if (tid < NS) {
        S.flag[tid] = 0u;
        S.bsum[tid] = 0ull;
    }
    __syncthreads();   // every wave reads entries that other waves copied

    // padding bytes of the header are part of the format (checked by the
    // first workgroup of each stream, spread over that stream's lanes)
    if (bid0 == 0) {
        const uint32_t lane = tid & 63u, wave = tid >> 6, row = lane >> 4;
        const uint32_t k = P == 1 ? sidx : row % P;
        const Lane ln = lane_stream<P>(a, k, 0);
        bool pad_bad = false;
        const uint32_t lane_in = wave * (64 / P) + (row / P) * 16 + (lane & 15u);
        for (uint64_t b = ln.table_pad_from + lane_in; b < ln.table_pad_to; b += NT / P) pad_bad |= ln.stream[b] != 0;
        for (uint64_t b = ln.nw_pad_from + lane_in; b < ln.nw_pad_to; b += NT / P) pad_bad |= ln.stream[b] != 0;
        if (pad_bad) atomicOr(&S.flag[P == 1 ? 0u : k], 1u);
    }

    // ---- the workgroup's tasks, one after the other (every wave of the
    // workgroup runs the same number; lanes past the last chunk decode
    // nothing)
    const uint32_t wave = __builtin_amdgcn_readfirstlane((uint32_t)tid >> 6);
    // Stream sizes (given, or read from the encoder's results) and the
    // codebooks' long-window offsets, once per workgroup: values common to
    // the workgroup, held in scalar registers.
    uint64_t s_words[NS];
    bool s_bad[NS];
    uint32_t s_long_sub[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const uint32_t si = P == 1 ? sidx : (uint32_t)q;
        const DecStream& d = a.st[si];
        uint64_t w = d.payload_words;
        bool sb = false;
        if (a.sizes) {
            const uint64_t b = a.sizes[si].bytes;
            const uint64_t bytes = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                                   __builtin_amdgcn_readfirstlane((uint32_t)b);
            const int32_t status = __builtin_amdgcn_readfirstlane(a.sizes[si].status);
            sb = status != 0 || bytes < d.header_bytes + 4 || ((bytes - d.header_bytes) & 3) != 0;
            w = sb ? 0 : (bytes - d.header_bytes) / 4;
        }
        s_words[q] = w;
        s_bad[q] = sb;
        s_long_sub[q] = __builtin_amdgcn_readfirstlane(d.cb->long_sub);
    }
    for (uint32_t bid = bid0; bid < a.wg_per_group; bid += a.wg_stride) {
    // The lane's geometry and stream are worked out again for every task:
    // the lane index comes from an asm statement the compiler cannot move
    // out of the loop, so nothing derived from it stays in a register from
    // one task to the next.
    const uint32_t lane = lane_index_fresh();
    const uint32_t row = lane >> 4, i16 = lane & 15u;
    const uint32_t k = P == 1 ? sidx : row % P;   // this lane's stream
    const uint32_t slot = P == 1 ? 0u : k;
    const uint32_t j = i16 & (G - 1);
    const uint64_t task = (uint64_t)bid * NW + wave;
    const uint64_t c = task * CPT + (row / P) * (16u >> LG) + (i16 >> LG);
    // this lane's stream's size and codebook field, picked by conditional
    // moves, not by an index into an array
    uint64_t my_words = 0;
    bool my_size_bad = false;
    uint32_t long_sub = 0;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const bool mine = P == 1 || (uint32_t)q == k;
        my_words = mine ? s_words[q] : my_words;
        my_size_bad = mine ? s_bad[q] : my_size_bad;
        long_sub = mine ? s_long_sub[q] : long_sub;
    }
    const Lane ln = lane_stream<P>(a, k, my_words);

    // ---- the chunk and its structure
    const bool valid = c < a.nc;
    bool bad = my_size_bad && valid;
    uint64_t sw = 0, wc = 0;
    uint32_t m = 0, N = 0;
    if (valid && !my_size_bad) {
        sw = c ? ln.table[c - 1] : 0;
        const uint64_t ew = ln.table[c];
        if (ew <= sw || ew > ln.payload_words) bad = true;
        wc = bad ? 0 : ew - sw;
        const uint32_t mc = (uint32_t)min<uint64_t>(a.chunk, a.n - c * a.chunk);
        m = lane_symbols<LG>(mc, j);
        N = ln.nw[(c << LG) + j];
        if ((m == 0) != (N == 0)) bad = true;
    }
    // the chunk's word counts must add up to its words; a bad lane stops its chunk
    if (group_sum<LG>(N) != (uint32_t)wc && valid && !my_size_bad) bad = true;
    const bool run = valid && group_sum<LG>(bad ? 1u : 0u) == 0;
    if (!run) {
        m = 0;
        N = 0;
        sw = 0;   // a chunk that is not decoded reads payload word 0 onwards (always in the buffer)
    }

    // ---- the group's ring: words of the chunk's payload, slot = word & (R - 1).
    // Loads are counted in words from a0 = sw rounded down to 4 (16-byte groups).
    uint32_t* const ring = &S.ring[wave][row][(i16 >> LG) * R];
    const uint64_t a0 = sw & ~uint64_t(3);
    const v4u* const grp = reinterpret_cast<const v4u*>(ln.payload + a0);
    // groups past the caller's payload are read as its last group (a0 lies in
    // the payload whenever the payload has a word)
    const uint64_t gall = ln.payload_words ? ((ln.payload_words - 1) >> 2) - (a0 >> 2) : 0;
    const uint32_t glast = (uint32_t)min<uint64_t>(gall, 0xFFFFFFFFull);
    // (a chunk that is not decoded reads 16 bytes of its codebook instead: every
    // load is issued, so the waits for them are counted exactly)
    // Loads past the chunk's words (and those of a chunk that is not decoded)
    // read 16 bytes of the codebook instead.
    const v4u* const safe = reinterpret_cast<const v4u*>(ln.cb);
    const uint32_t wend = (uint32_t)(sw - a0 + wc);   // the chunk's end, from a0
    auto load4 = [&](uint32_t word) -> v4u {   // this lane's 16 bytes of a group load at word a0 + word
        const uint32_t g = (word >> 2) + j;
        return *(run && word < wend ? grp + (g < glast ? g : glast) : safe);
    };
    const uint32_t slot0 = (uint32_t)a0 & (R - 1);
    auto put4 = [&](uint32_t word, const v4u& v) {
        *reinterpret_cast<v4u*>(&ring[(slot0 + word + 4 * j) & (R - 1)]) = v;
    };
    {
        const v4u v0 = load4(0), v1 = load4(4 * G), v2 = load4(8 * G), v3 = load4(12 * G);
        put4(0, v0);
        put4(4 * G, v1);
        put4(8 * G, v2);
        put4(12 * G, v3);
    }
    uint32_t wr = R;                            // next word to load (from a0)
    __builtin_amdgcn_wave_barrier();
    // two loads in flight: the one issued at a block's middle top-up, the one
    // issued at its end; each is written to the ring one block later
    uint32_t pa_at = 0, pb_at = 0;
    v4u pa = {0, 0, 0, 0}, pb = {0, 0, 0, 0};
    bool pa_on = false, pb_on = false;

    // ---- words 0 and 1
    uint32_t b0, n0, b1, n1;
    group_count<LG>(N >= 1, b0, n0);
    group_count<LG>(N >= 2, b1, n1);
    const uint32_t d0 = (uint32_t)(sw - a0);    // the chunk's first word, from a0
    // next word the group reads, from a0, plus the ring slot of a0 (so a
    // word's slot is the low bits of cs plus its count, one add)
    uint32_t cs = slot0 + d0 + n0 + n1;
    const uint32_t w0 = N >= 1 ? ring[(slot0 + d0 + b0) & (R - 1)] : 0u;
    const uint32_t w1 = N >= 2 ? ring[(slot0 + d0 + n0 + b1) & (R - 1)] : 0u;
    // Bit buffer: the lane's next avail = 64 - u bits, most significant first
    // (the two-word window with its used bits shifted out; u <= 63 while the
    // stream is valid).  "The first word is used up" is avail <= 32, i.e.
    // u >= 32; then a word comes in below the valid bits, shifted left by
    // u - 32 = u & 31, which is also the new u (a zero word once the lane has
    // read all its words).  vw, the words taken in (read or zero), is kept as
    // rp = N + 31 - vw, so that "a word is left to read" (vw < N) is rp >= 32
    // and a read is min(u, rp) >= 32, one comparison; 32 * (vw - 2) + u bits
    // are consumed.  Bit 7 of an entry marks a window that starts no code
    // word (its length field then is 0x90).
    uint64_t bb = ((uint64_t)w0 << 32) | w1;
    uint32_t u = 0;
    int32_t rp = (int32_t)N + 29;
    uint32_t inval = 0;

    // ---- decode, block by block
    // One block of 16 symbols: 8 pairs, each preceded by the group's reads.
    // FULL: every lane of the wave has the whole block (no symbol checks).
    // Ring top-up (group-uniform), after every 4 pairs: write the load issued
    // two top-ups ago to the ring, issue the next when the ring has room for
    // it (room counted with the loads in flight).  With 4G-word loads, a ring
    // of 16G words and 4 pairs reading at most 4G words between top-ups,
    // every word a pair reads has been written, and no write lands on a word
    // still to be read (the rule was checked exhaustively over consumption
    // patterns).  The top-up after a block's last pair comes before the
    // block's store, so waiting for a load gives the stores time to finish.
    auto top_up = [&](v4u& pv, uint32_t& pat, bool& pon) {
        if (pon) put4(pat, pv);
        // a load is issued every time; it is kept only when the ring has room
        // and the chunk has words there
        pon = wr + slot0 - cs <= R - 4 * G && wr < wend;
        pv = load4(wr);
        pat = wr;
        wr += pon ? 4 * G : 0u;
        __builtin_amdgcn_wave_barrier();
    };
    auto decode_block = [&](uint32_t t, auto full_c, uint32_t (&w)[4]) {
        constexpr bool FULL = decltype(full_c)::value;
        uint32_t ev[4];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (q == 4) top_up(pa, pa_at, pa_on);
            const uint32_t s0 = t * BLOCK + 2 * q;   // the pair's first symbol in the lane
            const bool act = FULL || s0 < m;
            const bool fetch = min((int32_t)u, act ? rp : 0) >= 32;
            uint32_t bf, nf;
            group_count<LG>(fetch, bf, nf);
            const uint32_t word = ring[(cs + bf) & (R - 1)];
            // avail >= 1 before a pair (a pair takes at most 32 of > 32 bits): u <= 63
            const uint32_t u31 = u & 31u;
            bb |= (uint64_t)(fetch ? word : 0u) << u31;
            if (FULL || act) {
                rp -= (int32_t)(u >> 5);   // (one word taken in when u >= 32)
                u = u31;
            }
            cs += nf;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bool use = FULL || s0 + h < m;
                const uint32_t idx = dec_index((uint32_t)(bb >> 32), long_sub);
                uint32_t e;
                if constexpr (P == 1) e = S.dec[idx];
                else e = S.dec[k][idx];
                if constexpr (!FULL) e = use ? e : 0u;
                bb <<= (e & 63u);   // (len <= 16; bits 8.. hold the symbol)
                u += e & 0xFFu;
                const int x = 2 * q + h;
                ev[x & 3] = e;
                if ((x & 3) == 3) w[x >> 2] = syms4(ev);
            }
            inval |= ev[(2 * q) & 3] | ev[(2 * q + 1) & 3];   // bit 7: no code word starts here
        }
        top_up(pb, pb_at, pb_on);
    };
    uint32_t mmax = m, mmin = m;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mmax = max(mmax, (uint32_t)__shfl_xor(mmax, o, 64));
        mmin = min(mmin, (uint32_t)__shfl_xor(mmin, o, 64));
    }
    const uint32_t nblk = (mmax + BLOCK - 1) / BLOCK, nfull = mmin / BLOCK;
    // Output addresses: the task's first element (common to the wave, so the
    // bases below are scalar) plus the lane's 32-bit offset from it (a task
    // spans at most 4 * 65536 elements).
    const uint64_t task_e0 = task * CPT * (uint64_t)a.chunk;
    const uint32_t lane_e0 = ((row / P) * (16u >> LG) + (i16 >> LG)) * a.chunk + j * BLOCK;  // lane's block 0
    uint8_t* const out_t = P == 1 ? ln.out + task_e0 : nullptr;   // OUT_PLANES
    uint8_t* const merged_t = a.merged + (uint64_t)P * task_e0;    // OUT_U16, OUT_U16_XOR, OUT_U32
    const uint8_t* const w0_t = a.w0 + 2 * task_e0;                // OUT_U16_XOR
    // The output of block t: 16 symbols of block tG + j of the chunk (FULL:
    // every lane's block is whole).  Whole blocks go out as non-temporal
    // stores (the decode never reads its output back; measured 2.5 % faster
    // than plain stores on 1 GiB of int8).
    // (x0: FULL, OUT_U16_XOR: the block's 16 bytes of the other snapshot,
    // loaded before the block's ring loads so that their wait does not drain
    // them)
    auto store_block = [&](uint32_t t, const uint32_t (&w)[4], auto full_c, const v4u& x0) {
        constexpr bool FULL = decltype(full_c)::value;
        const uint32_t cnt = FULL ? BLOCK : (m > t * BLOCK ? min(BLOCK, m - t * BLOCK) : 0u);
        const uint32_t e0 = lane_e0 + (t << LG) * BLOCK;
        if constexpr (OUT == DEC_OUT_PLANES) {
            if (FULL || cnt == BLOCK) {
                v4u v;
                v.x = w[0];
                v.y = w[1];
                v.z = w[2];
                v.w = w[3];
                __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(out_t + e0));
            } else {
                for (uint32_t x = 0; x < cnt; ++x) out_t[e0 + x] = (uint8_t)(w[x >> 2] >> (8 * (x & 3)));
            }
        } else {
            // every lane takes part in the exchanges; the lanes of one element
            // group have the same cnt
            if constexpr (OUT == DEC_OUT_U16 || OUT == DEC_OUT_U16_XOR) {
                v4u v = restore_u16(w, k);
                const uint32_t at = 2 * e0 + 16 * k;
                if (FULL || cnt == BLOCK) {
                    if constexpr (OUT == DEC_OUT_U16_XOR) v ^= FULL ? x0 : *reinterpret_cast<const v4u*>(w0_t + at);
                    __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(merged_t + at));
                }
            } else {
                const v4u v = restore_u32(w, k);
                if (FULL || cnt == BLOCK) __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(merged_t + 4 * e0 + 16 * k));
            }
            if (!FULL && cnt && cnt < BLOCK) {
                // the tensor's last block: byte P-1-k of each element (plane k holds byte P-1-k)
                for (uint32_t x = 0; x < cnt; ++x) {
                    const uint32_t at = P * (e0 + x) + (P - 1 - k);
                    const uint8_t sym = (uint8_t)(w[x >> 2] >> (8 * (x & 3)));
                    merged_t[at] = OUT == DEC_OUT_U16_XOR ? (uint8_t)(sym ^ w0_t[at]) : sym;
                }
            }
        }
    };
    // A wave whose lanes all have only whole blocks (every wave but those of
    // the tensor's last chunk) runs a loop of whole blocks: every lane ends
    // each block with the same memory operations (two ring loads, one store),
    // so the compiler's waits for a ring load count the store issued after
    // the older load and leave it in flight.  (With the general blocks in
    // the same loop the store could not be counted, and the wait also drained
    // the newer ring load.)  The other waves take the general block for all
    // their blocks: two loops, one taken, so their registers are not live at
    // the same time.
    if (nfull == nblk) {
        for (uint32_t t = 0; t < nblk; ++t) {
            uint32_t w[4];
            v4u x0 = {0, 0, 0, 0};
            if constexpr (OUT == DEC_OUT_U16_XOR)
                x0 = *reinterpret_cast<const v4u*>(w0_t + 2 * (lane_e0 + (t << LG) * BLOCK) + 16 * k);
            decode_block(t, std::true_type{}, w);
            store_block(t, w, std::true_type{}, x0);
        }
    } else {
        for (uint32_t t = 0; t < nblk; ++t) {
            uint32_t w[4];
            decode_block(t, std::false_type{}, w);
            store_block(t, w, std::false_type{}, v4u{0, 0, 0, 0});
        }
    }
    // ---- the lane's end: every word read, the last one needed, zero padding
    uint32_t bits = 0;
    if (run && m) {
        const uint32_t vw = (uint32_t)((int32_t)N + 31 - rp);
        bits = 32 * (vw - 2) + u;
        if ((inval & 0x80u) || vw < N || bits > 32 * N || bits <= 32 * (N - 1)) bad = true;
        const uint32_t rest = 32 * N - bits;   // padding bits: the next ones in the buffer
        if (!bad && rest && (bb >> (64 - rest)) != 0) bad = true;
    }

    // ---- the task's status and bits, per stream of the workgroup
    if (bad) atomicOr(&S.flag[slot], 1u);
    {
        // bits of the lanes decoded without fault, summed per row (one stream
        // per row; a lane has at most 4096 symbols of at most 16 bits, so the
        // sum fits 32 bits)
        const uint32_t v = group_sum<4>((run && !bad) ? bits : 0u);
        if (i16 == 0 && v) atomicAdd(&S.bsum[slot], (unsigned long long)v);
    }
    }   // the workgroup's tasks

    // ---- status, accounting, exit
    __syncthreads();
    const uint32_t tid_end = wave * 64 + lane_index_fresh();
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        if (tid_end == (uint32_t)q) {
            const DecStream& d = a.st[P == 1 ? sidx : (uint32_t)q];
            if (S.bsum[q]) atomicAdd(reinterpret_cast<unsigned long long*>(&d.ws->bits), S.bsum[q]);
            if (S.flag[q]) atomicCAS(&d.ws->status, 0, (int32_t)LECB_ERR_CORRUPT);
        }
    }
    if (tid_end == 0) {
        __threadfence();
        WsHeader* ws0 = a.st[0].ws;
        const uint32_t done = __hip_atomic_fetch_add(&ws0->exit_count, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            for (uint32_t s = 0; s < a.nstreams; ++s) {
                DecStream e = a.st[s];
                if (a.sizes) {
                    const uint64_t bytes = a.sizes[s].bytes;
                    e.payload_words = bytes >= e.header_bytes ? (bytes - e.header_bytes) / 4 : 0;
                }
                const uint64_t bits_all = __hip_atomic_load(&e.ws->bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int32_t st = __hip_atomic_load(&e.ws->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t W = e.table[a.nc - 1];
                e.res->bytes = e.header_bytes + 4 * W;
                e.res->payload_bits = bits_all;
                e.res->status = (st == 0 && W != e.payload_words) ? (int32_t)LECB_ERR_CORRUPT : st;
                e.res->reserved = 0;
                e.ws->bits = 0;
                e.ws->status = 0;
            }
            __threadfence();
            __hip_atomic_store(&ws0->exit_count, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int NT, int P, int OUT>
const void* kernel_of(uint32_t lg) {
    switch (lg) {
        case 0: return reinterpret_cast<const void*>(&decode_kernel<NT, P, OUT, 0>);
        case 1: return reinterpret_cast<const void*>(&decode_kernel<NT, P, OUT, 1>);
        case 2: return reinterpret_cast<const void*>(&decode_kernel<NT, P, OUT, 2>);
        case 3: return reinterpret_cast<const void*>(&decode_kernel<NT, P, OUT, 3>);
        case 4: return reinterpret_cast<const void*>(&decode_kernel<NT, P, OUT, 4>);
        default: return nullptr;
    }
}

// Workgroups of one decode kernel resident on a CU (asked once per device and
// kernel; concurrent first calls store the same value).
constexpr int DEC_VARIANTS = 11;
template <int NT, int P, int OUT>
uint64_t resident_per_cu(int variant, uint32_t lg) {
    static std::atomic<int> cached[MAX_DEVICES][DEC_VARIANTS][5];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return 1;
    int nb = cached[dev][variant][lg].load(std::memory_order_relaxed);
    if (!nb) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel_of<NT, P, OUT>(lg), NT, 0) != hipSuccess || nb <= 0)
            nb = 1;
        cached[dev][variant][lg].store(nb, std::memory_order_relaxed);
    }
    return (uint64_t)nb;
}

// Launch with wg_tasks workgroup tasks per stream (OUT_PLANES: one stream per
// workgroup, `groups` streams) or in all (groups = 1): as many workgroups as
// the CUs hold at once (never more than the tasks), each looping over its
// tasks.
template <int NT, int P, int OUT>
hipError_t launch(DecArgs& a, int variant, uint32_t lg, uint64_t wg_tasks, uint32_t groups, uint64_t cus,
                  hipStream_t hs) {
    if (lg > 4) return hipErrorInvalidValue;
    if (wg_tasks == 0 || wg_tasks > 0xFFFFFFFFull) return hipErrorInvalidValue;
    const uint64_t resident = cus * resident_per_cu<NT, P, OUT>(variant, lg);
    const uint64_t per_group = std::max<uint64_t>(1, resident / groups);
    a.wg_per_group = (uint32_t)wg_tasks;
    a.wg_stride = (uint32_t)std::min<uint64_t>(wg_tasks, per_group);
    const uint32_t wgs = a.wg_stride * groups;
    switch (lg) {
        case 0: hipLaunchKernelGGL((decode_kernel<NT, P, OUT, 0>), dim3(wgs), dim3(NT), 0, hs, a); break;
        case 1: hipLaunchKernelGGL((decode_kernel<NT, P, OUT, 1>), dim3(wgs), dim3(NT), 0, hs, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<NT, P, OUT, 2>), dim3(wgs), dim3(NT), 0, hs, a); break;
        case 3: hipLaunchKernelGGL((decode_kernel<NT, P, OUT, 3>), dim3(wgs), dim3(NT), 0, hs, a); break;
        default: hipLaunchKernelGGL((decode_kernel<NT, P, OUT, 4>), dim3(wgs), dim3(NT), 0, hs, a); break;
    }
    return hipSuccess;
}

}  // namespace

int launch_decode(const DecodeLaunch& L, void* stream) {
    DecArgs a{};
    const uint64_t tb = table_bytes(L.nc), cb = count_bytes(L.nc, L.chunk);
    const uint32_t G = lanes_per_chunk(L.chunk);
    const uint32_t lg = (uint32_t)ilog2(G);
    a.chunk = L.chunk;
    a.n = L.n;
    a.nc = L.nc;
    a.nstreams = L.nstreams;
    a.sizes = L.dev_sizes;
    a.merged = L.merged;
    a.w0 = L.w0;
    if (L.nstreams < 1 || L.nstreams > 4) return LECB_ERR_INVALID_ARG;
    for (int s = 0; s < L.nstreams; ++s) {
        DecStream& st = a.st[s];
        st.table = reinterpret_cast<const uint32_t*>(L.stream_base[s]);
        st.nw = reinterpret_cast<const uint16_t*>(L.stream_base[s] + tb);
        st.payload = reinterpret_cast<const uint32_t*>(L.stream_base[s] + tb + cb);
        st.payload_words = L.dev_sizes ? 0 : (L.stream_bytes[s] - tb - cb) / 4;
        st.cb = L.cb[s];
        st.header_bytes = tb + cb;
        st.stream = L.stream_base[s];
        st.table_pad_from = 4 * L.nc;
        st.table_pad_to = tb;
        st.nw_pad_from = tb + 2 * L.nc * G;
        st.nw_pad_to = tb + cb;
        st.out = L.out[s];
        st.res = L.res[s];
        st.ws = L.ws[s];
    }
    const uint64_t cus = (uint64_t)device_cu_count();
    if (cus == 0) return LECB_ERR_HIP;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    // Workgroup size: 16 waves (12 for two planes, 6 for four: the tables are
    // one copy per workgroup) when the tasks give every CU such a workgroup,
    // else 4 waves, so that small inputs still spread over the CUs.
    if (L.out_kind == DEC_OUT_PLANES) {
        const uint64_t cpt = 4 * (16 >> lg);
        const uint64_t tasks = (L.nc + cpt - 1) / cpt;
        const bool big = tasks * (uint64_t)L.nstreams >= cus * 16;
        const uint64_t nw = big ? 16 : 4;
        const uint64_t wg_tasks = (tasks + nw - 1) / nw;
        const uint32_t ns = (uint32_t)L.nstreams;
        e = big ? launch<1024, 1, DEC_OUT_PLANES>(a, 0, lg, wg_tasks, ns, cus, hs)
                : launch<256, 1, DEC_OUT_PLANES>(a, 1, lg, wg_tasks, ns, cus, hs);
    } else if (L.out_kind == DEC_OUT_U16 || L.out_kind == DEC_OUT_U16_XOR) {
        if (L.nstreams != 2 || !L.merged || (L.out_kind == DEC_OUT_U16_XOR && !L.w0)) return LECB_ERR_INVALID_ARG;
        // (two planes need more registers per lane: 12-wave workgroups; when
        // one 16-wave workgroup per CU holds every task, those instead, so
        // that every SIMD gets the same number of waves)
        const uint64_t cpt = 2 * (16 >> lg);
        const uint64_t tasks = (L.nc + cpt - 1) / cpt;
        const bool big = tasks >= cus * 12;
        const bool one_round = big && tasks <= cus * 16;
        const uint64_t nw = one_round ? 16 : big ? 12 : 4;
        const uint64_t wg_tasks = (tasks + nw - 1) / nw;
        if (L.out_kind == DEC_OUT_U16)
            e = one_round ? launch<1024, 2, DEC_OUT_U16>(a, 8, lg, wg_tasks, 1, cus, hs)
                : big     ? launch<768, 2, DEC_OUT_U16>(a, 2, lg, wg_tasks, 1, cus, hs)
                          : launch<256, 2, DEC_OUT_U16>(a, 3, lg, wg_tasks, 1, cus, hs);
        else
            e = one_round ? launch<1024, 2, DEC_OUT_U16_XOR>(a, 9, lg, wg_tasks, 1, cus, hs)
                : big     ? launch<768, 2, DEC_OUT_U16_XOR>(a, 4, lg, wg_tasks, 1, cus, hs)
                          : launch<256, 2, DEC_OUT_U16_XOR>(a, 5, lg, wg_tasks, 1, cus, hs);
    } else if (L.out_kind == DEC_OUT_U32) {
        if (L.nstreams != 4 || !L.merged) return LECB_ERR_INVALID_ARG;
        // (four tables in LDS: 6-wave workgroups; one 16-wave workgroup per CU
        // when that holds every task)
        const uint64_t cpt = 16 >> lg;
        const uint64_t tasks = (L.nc + cpt - 1) / cpt;
        const bool big = tasks >= cus * 6;
        const bool one_round = big && tasks <= cus * 16;
        const uint64_t nw = one_round ? 16 : big ? 6 : 4;
        const uint64_t wg_tasks = (tasks + nw - 1) / nw;
        e = one_round ? launch<1024, 4, DEC_OUT_U32>(a, 10, lg, wg_tasks, 1, cus, hs)
            : big     ? launch<384, 4, DEC_OUT_U32>(a, 6, lg, wg_tasks, 1, cus, hs)
                      : launch<256, 4, DEC_OUT_U32>(a, 7, lg, wg_tasks, 1, cus, hs);
    } else {
        return LECB_ERR_INVALID_ARG;
    }
    if (e != hipSuccess) return LECB_ERR_INVALID_ARG;
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

}  // namespace lecb
