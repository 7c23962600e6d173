// Huffman decode of stream format v2 back to bytes, and back to 16-bit or
// 32-bit elements when the byte groups are decoded together.
//
// Reverse path of "Lossless Compression for LLM Tensor Incremental
// Snapshots", Technical framework (read, Huffman-decode, restore the byte
// groups); the independent parallel tasks of its Key design item 3 are the
// decode units: unit j of a chunk is its symbols [256j, 256j + 256), and the
// stored code-bit counts of the chunk's units give every unit's first bit.
//
// One lane per unit and byte plane.  P planes of the same element are coded
// as P streams whose units cover the same symbols, so the P lanes of a unit
// (neighbouring lanes of one wave) produce the P bytes of the same 256
// elements in lockstep:
//   * P = 1, OUT_PLANES: each stream's units in workgroups of their own, one
//     byte per symbol written to that stream's output;
//   * P = 2, OUT_U16 / OUT_U16_XOR: lane 2u decodes the high plane and lane
//     2u + 1 the low plane of unit u; after every 16 symbols the pair swaps
//     half of its bytes (lane exchanges) and each lane stores 8 restored
//     16-bit words (16 bytes), XORed with the other snapshot for a delta;
//   * P = 4, OUT_U32: lanes 4u..4u+3 decode planes 0..3 (bytes 3..0 of the
//     32-bit elements) of unit u; after every 16 symbols the quad transposes
//     its words and each lane stores 4 restored elements.
//
// Per lane:
//   1. its unit's first bit = the sum of the bit counts of the chunk's
//      earlier units (a segmented scan over the workgroup's lanes: a chunk's
//      units never straddle workgroups);
//   2. decode the unit's symbols (256, fewer only at the end of the tensor)
//      from that bit; the unit must end exactly at first bit + its count, and
//      the unit holding the chunk's last symbol checks the zero padding to
//      the end of the chunk's last word.
//
// Bit reader: a window of two payload words and a bit offset into it; before
// every pair of code words the window slides by one word when its first word
// is used up (no branch).  Afterwards the offset is below 32, so the window
// holds >= 33 bits, enough for two code words of at most 16 bits.  The words
// come from a per-lane ring of 16 payload words in LDS; the ring is topped up
// on a fixed schedule (every 4 refills) by one 32-byte global load whose data
// go into the ring at the next top-up, so the decode loop never waits on
// global memory.  Ring slot q of lane L sits at ring[q][L]: each lane has its
// own bank.
//
// A code word of at most LUT_BITS bits is one LDS lookup, a longer one a
// lookup in a second table.  Every structural rule of the format is checked;
// a violation sets status CORRUPT.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "lecb_internal.hpp"

namespace lecb {

namespace {

constexpr uint32_t RING = 16;   // payload words per lane in LDS
constexpr uint32_t UNIT = LECB_UNIT_SYMBOLS;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

struct DecStream {
    const uint32_t* table;
    const uint16_t* ulen;
    const uint32_t* payload;
    uint64_t payload_words;   // words present in the caller's buffer
    const DeviceCodebook* cb;
    uint64_t header_bytes;
    uint64_t table_pad_from, table_pad_to;   // stream bytes that must be zero
    uint64_t ulen_pad_from, ulen_pad_to;
    const uint8_t* stream;
    uint8_t* out;             // OUT_PLANES: the decoded bytes of this stream
    lecb_result* res;
    WsHeader* ws;
};

struct DecArgs {
    const lecb_result* sizes;  // non-null: stream k's size is sizes[k].bytes (an encoder's result)
    uint32_t chunk;
    uint32_t log2k;
    uint64_t n;
    uint64_t nc;
    uint32_t wg_per_group;     // OUT_PLANES: workgroups of one stream; stream = blockIdx.x / wg_per_group
    uint32_t nstreams;
    uint8_t* merged;           // OUT_U16, OUT_U16_XOR, OUT_U32: the restored elements
    const uint8_t* w0;         // OUT_U16_XOR: the other snapshot (element i ^ restored i is written)
    DecStream st[4];
};

// One stream's tables in a workgroup with one stream per workgroup: the
// decode table and the canonical tables of the longer code words.
template <int NT>
struct SharedOne {
    uint16_t lut[1][LUT_SIZE];   // (sym << 8) | len of the code words of at most LUT_BITS bits
    uint16_t lut2[LUT2_SIZE];    // the same for the longer code words
    alignas(16) uint32_t ring[RING][NT];
};
// P streams in every workgroup: P first tables (code words longer than
// LUT_BITS -- rare in byte planes -- read the second table of the device
// codebook in memory).  With P = 2 and 1024 lanes this is exactly 80 KiB, so
// two workgroups fill a CU's LDS.
template <int NT, int P>
struct SharedMany {
    uint16_t lut[P][LUT_SIZE];
    alignas(16) uint32_t ring[RING][NT];
};
template <int NT, int P>
using Shared = std::conditional_t<P == 1, SharedOne<NT>, SharedMany<NT, P>>;

template <int NT>
struct Reader {
    uint32_t* ring;      // &ring[0][lane]
    const uint32_t* p;   // payload
    uint64_t sw;         // chunk's first payload word
    uint64_t gmax;       // last readable 4-word group of the payload
    uint32_t sh;         // sw mod RING
    uint32_t rq;         // sh + index (relative to sw) of the word held in nextw;
                         // w1 is the word before it, w0 the one before that
    uint32_t wr;         // next word (relative to sw) to load; sw + wr is a multiple of 8
    uint32_t w0, w1;     // 64-bit window; the next bit is bit `off` from the top of w0
    uint32_t off;        // < 32 after refill()
    uint32_t nextw;
    v4u pa, pb;          // loaded, not yet in the ring
    bool pend;

    __device__ inline uint32_t& slot(uint32_t w) {  // w relative to sw
        return ring[((w + sh) & (RING - 1)) * NT];
    }
    __device__ inline uint32_t rd() const { return rq - sh; }
    __device__ inline v4u ld4(uint64_t g) const {
        return *reinterpret_cast<const v4u*>(p + 4 * (g < gmax ? g : gmax));
    }
    __device__ inline void put8(uint32_t w, const v4u& x, const v4u& y) {
        uint32_t* s = &slot(w);  // w..w+7 are consecutive slots (sw + w is a multiple of 8)
        s[0 * NT] = x.x;
        s[1 * NT] = x.y;
        s[2 * NT] = x.z;
        s[3 * NT] = x.w;
        s[4 * NT] = y.x;
        s[5 * NT] = y.y;
        s[6 * NT] = y.z;
        s[7 * NT] = y.w;
    }
    // Ring top-up: commit the previous load, issue the next one when there is
    // room.  Between two top-ups at most 4 words leave the ring, and after a
    // top-up at least 5 committed words lie at or after rd, so the word read
    // by refill() is always in the ring.
    __device__ inline void tick() {
        if (pend) {
            put8(wr - 8, pa, pb);
            pend = false;
        }
        if (wr - rd() <= 8) {
            const uint64_t g = (sw + wr) >> 2;
            pa = ld4(g);
            pb = ld4(g + 1);
            wr += 8;
            pend = true;
        }
    }
    // Position the reader at bit `bit` of the chunk (synchronous 16-word load).
    __device__ inline void start(uint32_t bit) {
        const uint32_t word = bit >> 5;
        const uint64_t a = (sw + word) & ~uint64_t(7);
        wr = (uint32_t)(a - sw);
        put8(wr, ld4(a >> 2), ld4((a >> 2) + 1));
        put8(wr + 8, ld4((a >> 2) + 2), ld4((a >> 2) + 3));
        wr += 16;
        pend = false;
        w0 = slot(word);
        w1 = slot(word + 1);
        rq = word + 2 + sh;
        nextw = ring[(rq & (RING - 1)) * NT];
        off = bit & 31;
    }
    // The next 32 bits, MSB first (all of them valid while off <= 32).
    __device__ inline uint32_t peek() const {
        return (uint32_t)(((((uint64_t)w0 << 32) | w1) << off) >> 32);
    }
    // bits consumed, relative to the chunk start
    __device__ inline uint32_t pos() const { return 32 * (rd() - 2) + off; }
    // Slide the window by one word once its first word is used up.  No
    // branch; afterwards off < 32 (the caller never lets off reach 64).
    __device__ inline void refill() {
        const bool take = off >= 32;
        w0 = take ? w1 : w0;
        w1 = take ? nextw : w1;
        off &= 31;
        rq += take ? 1u : 0u;
        nextw = ring[(rq & (RING - 1)) * NT];
    }
};

// What a lane needs of its stream (selected per lane when a workgroup holds
// several streams).
struct Lane {
    const uint32_t* table;
    const uint16_t* ulen;
    const uint32_t* payload;
    uint64_t payload_words;
    const DeviceCodebook* cb;
    uint8_t* out;
    const uint8_t* stream;
    uint64_t table_pad_from, table_pad_to, ulen_pad_from, ulen_pad_to;
};

template <int P>
__device__ inline Lane lane_stream(const DecArgs& a, uint32_t k, uint64_t payload_words) {
    Lane l;
#define LECB_PICK(field, expr)                                            \
    if constexpr (P == 1) {                                               \
        l.field = a.st[k].expr;                                           \
    } else if constexpr (P == 2) {                                        \
        l.field = k ? a.st[1].expr : a.st[0].expr;                        \
    } else {                                                              \
        l.field = k & 2 ? (k & 1 ? a.st[3].expr : a.st[2].expr)           \
                        : (k & 1 ? a.st[1].expr : a.st[0].expr);          \
    }
    LECB_PICK(table, table)
    LECB_PICK(ulen, ulen)
    LECB_PICK(payload, payload)
    LECB_PICK(cb, cb)
    LECB_PICK(out, out)
    LECB_PICK(stream, stream)
    LECB_PICK(table_pad_from, table_pad_from)
    LECB_PICK(table_pad_to, table_pad_to)
    LECB_PICK(ulen_pad_from, ulen_pad_from)
    LECB_PICK(ulen_pad_to, ulen_pad_to)
#undef LECB_PICK
    l.payload_words = payload_words;
    return l;
}

// Next code word as (sym << 8) | len, len in 1..16, from the next 32 bits
// `top`.  An invalid code word yields len 16 and sets `inval`.  A code word
// of at most LUT_BITS bits is one probe of the first table, a longer one one
// probe of the second (which always holds every longer code word: at most 256
// of them, each covering at most 2^(16 - 13) = 8 of its entries).
template <int P, typename S>
__device__ inline uint32_t lookup(const S& sh, const uint16_t* lut, const DeviceCodebook* cb, uint32_t base2,
                                  uint32_t top, uint32_t& inval) {
    uint32_t e = lut[top >> (32 - LUT_BITS)];
    if (e == 0) {
        const uint32_t i = (top >> 16) - base2;
        if constexpr (P == 1) e = i < (uint32_t)LUT2_SIZE ? sh.lut2[i] : 0u;
        else e = i < (uint32_t)LUT2_SIZE ? cb->lut2[i] : 0u;
        if (e == 0) {
            inval = 1;
            e = 16;
        }
    }
    return e;
}

// The symbols (byte 1) of four table entries as one little-endian word:
// two byte permutes gather the pairs, a third joins them.
__device__ inline uint32_t syms4(const uint32_t (&e)[4]) {
    const uint32_t p01 = __builtin_amdgcn_perm(e[1], e[0], 0x0c0c0501u);
    const uint32_t p23 = __builtin_amdgcn_perm(e[3], e[2], 0x0c0c0501u);
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}

// 16 restored 16-bit words from the high-plane bytes of 16 symbols (lane 2u,
// w[0..3]) and the low-plane bytes (lane 2u + 1): the pair swaps half of its
// words, then lane 2u builds words 0..7 and lane 2u + 1 words 8..15
// (little-endian: low byte first).
__device__ inline v4u restore_u16(const uint32_t (&w)[4], uint32_t odd) {
    const uint32_t s0 = __shfl_xor(odd ? w[0] : w[2], 1, 64);
    const uint32_t s1 = __shfl_xor(odd ? w[1] : w[3], 1, 64);
    const uint32_t h0 = odd ? s0 : w[0], h1 = odd ? s1 : w[1];
    const uint32_t l0 = odd ? w[2] : s0, l1 = odd ? w[3] : s1;
    v4u o;
    o.x = __builtin_amdgcn_perm(h0, l0, 0x05010400u);
    o.y = __builtin_amdgcn_perm(h0, l0, 0x07030602u);
    o.z = __builtin_amdgcn_perm(h1, l1, 0x05010400u);
    o.w = __builtin_amdgcn_perm(h1, l1, 0x07030602u);
    return o;
}

// 16 restored 32-bit elements from four lanes q = 0..3 holding the bytes of
// planes 0..3 (element bytes 3..0) of 16 symbols: lane q gathers word q of
// every plane (three exchanges) and builds elements 4q..4q+3.
__device__ inline v4u restore_u32(const uint32_t (&w)[4], uint32_t q) {
    uint32_t x0 = 0, x1 = 0, x2 = 0, x3 = 0;  // word q of planes 0..3
#pragma unroll
    for (uint32_t r = 0; r < 4; ++r) {
        // round r: lane q reads lane (q + r) & 3, which sends its word (self - r) & 3
        const uint32_t src = (q + r) & 3u;
        const uint32_t want = (q - r) & 3u;
        // (masks rather than an index: the words stay in registers)
        const uint32_t mine = (w[0] & (0u - (uint32_t)(want == 0))) | (w[1] & (0u - (uint32_t)(want == 1))) |
                              (w[2] & (0u - (uint32_t)(want == 2))) | (w[3] & (0u - (uint32_t)(want == 3)));
        const uint32_t got = r ? __shfl(mine, (int)((threadIdx.x & ~3u) | src), 64) : mine;
        x0 = src == 0 ? got : x0;
        x1 = src == 1 ? got : x1;
        x2 = src == 2 ? got : x2;
        x3 = src == 3 ? got : x3;
    }
    // element k: bytes [x3[k], x2[k], x1[k], x0[k]] (little-endian)
    const uint32_t a01 = __builtin_amdgcn_perm(x0, x1, 0x05010400u);  // x1_0 x0_0 x1_1 x0_1
    const uint32_t b01 = __builtin_amdgcn_perm(x0, x1, 0x07030602u);  // x1_2 x0_2 x1_3 x0_3
    const uint32_t a23 = __builtin_amdgcn_perm(x2, x3, 0x05010400u);  // x3_0 x2_0 x3_1 x2_1
    const uint32_t b23 = __builtin_amdgcn_perm(x2, x3, 0x07030602u);
    v4u o;
    o.x = __builtin_amdgcn_perm(a01, a23, 0x05040100u);  // x3_0 x2_0 x1_0 x0_0
    o.y = __builtin_amdgcn_perm(a01, a23, 0x07060302u);
    o.z = __builtin_amdgcn_perm(b01, b23, 0x05040100u);
    o.w = __builtin_amdgcn_perm(b01, b23, 0x07060302u);
    return o;
}

template <int NT, int P>
__device__ inline const uint16_t* lut_of(const Shared<NT, P>& S, uint32_t k) {
    return &S.lut[P == 1 ? 0 : k][0];
}

// 64 VGPRs at most: two 1024-lane workgroups (8 waves per SIMD) fit a CU.
template <int NT, int P, int OUT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8, 8))) void decode_kernel(DecArgs a) {
    static_assert(P == 1 || OUT != DEC_OUT_PLANES, "plane outputs decode one stream per workgroup");
    __shared__ __attribute__((aligned(16))) Shared<NT, P> S;
    const int tid = threadIdx.x;

    // ---- which stream, unit and chunk this lane decodes
    const uint32_t sidx = P == 1 ? blockIdx.x / a.wg_per_group : 0u;     // P == 1: stream of the workgroup
    const uint32_t bid = P == 1 ? blockIdx.x - sidx * a.wg_per_group : blockIdx.x;
    const uint32_t k = P == 1 ? sidx : (uint32_t)tid & (P - 1);           // this lane's stream
    const uint64_t u = P == 1 ? (uint64_t)bid * NT + tid : ((uint64_t)bid * NT + tid) / P;
    // stream sizes: given, or read from the encoder's results (this lane's
    // stream picked by conditional moves, not by an index into an array)
    uint64_t my_words = 0;
    bool my_size_bad = false;
#pragma unroll
    for (int q = 0; q < (P == 1 ? 1 : P); ++q) {
        const uint32_t s = P == 1 ? sidx : (uint32_t)q;
        const DecStream& d = a.st[s];
        uint64_t w = d.payload_words;
        bool sb = false;
        if (a.sizes) {
            const uint64_t bytes = a.sizes[s].bytes;
            sb = a.sizes[s].status != 0 || bytes < d.header_bytes + 4 || ((bytes - d.header_bytes) & 3) != 0;
            w = sb ? 0 : (bytes - d.header_bytes) / 4;
        }
        const bool mine = P == 1 || (uint32_t)q == k;
        my_words = mine ? w : my_words;
        my_size_bad = mine ? sb : my_size_bad;
    }
    const Lane ln = lane_stream<P>(a, k, my_words);
    // ---- tables
    {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const v4u* src = reinterpret_cast<const v4u*>(a.st[P == 1 ? sidx : (uint32_t)q].cb->lut);
            v4u* dst = reinterpret_cast<v4u*>(&S.lut[q][0]);
            constexpr int NV = LUT_SIZE * 2 / 16;
            for (int i = tid; i < NV; i += NT) dst[i] = src[i];
        }
        if constexpr (P == 1) {
            const v4u* src2 = reinterpret_cast<const v4u*>(a.st[sidx].cb->lut2);
            v4u* dst2 = reinterpret_cast<v4u*>(S.lut2);
            for (int i = tid; i < LUT2_SIZE * 2 / 16; i += NT) dst2[i] = src2[i];
        }
    }
    const uint32_t base2 = ln.cb->lut2_base;

    // ---- unit geometry and the stream's structure around it
    const uint32_t K = 1u << a.log2k;
    const uint64_t c = u >> a.log2k;
    const uint32_t j = (uint32_t)(u & (K - 1));
    const bool active = c < a.nc && !my_size_bad;
    bool bad = my_size_bad && c < a.nc;
    uint64_t sw = 0, wc = 0;
    uint32_t m_c = 0, cnt = 0, my_bits = 0;
    if (active) {
        sw = c ? ln.table[c - 1] : 0;
        const uint64_t ew = ln.table[c];
        if (ew <= sw || ew > ln.payload_words || ew - sw > a.chunk / 2) bad = true;
        wc = bad ? 0 : ew - sw;
        m_c = (uint32_t)min<uint64_t>(a.chunk, a.n - c * a.chunk);
        cnt = m_c > j * UNIT ? min(m_c - j * UNIT, UNIT) : 0u;
        my_bits = ln.ulen[u];
        if (my_bits < cnt || my_bits > 16 * cnt) bad = true;
    }
    // first bit of every unit: exclusive sum of the bit counts of the chunk's
    // earlier units of the same stream (segments of K*P lanes; the ring's first
    // row holds the sums until the decode starts)
    uint32_t* const scan = &S.ring[0][0];
    scan[tid] = my_bits;
    __syncthreads();
    const uint32_t seg = K * P;  // lanes of one chunk (all streams); divides NT
    const uint32_t in_seg = (uint32_t)tid & (seg - 1);
    for (uint32_t o = P; o < seg; o <<= 1) {
        const uint32_t v = in_seg >= o ? scan[tid - o] : 0u;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    const uint32_t first_bit = scan[tid] - my_bits;
    const uint32_t chunk_bits = scan[(tid - in_seg) + (K - 1) * P + (tid & (P - 1))];
    __syncthreads();  // the ring is written from here on
    if (active && !bad) {
        // the chunk's bits fill its words to within one word
        if (chunk_bits == 0 || (uint64_t)chunk_bits > 32 * wc || (uint64_t)chunk_bits + 32 <= 32 * wc) bad = true;
    }

    // padding bytes of the header are part of the format (checked by the
    // first workgroup of each stream, spread over that stream's lanes)
    if (bid == 0) {
        const uint32_t lane_in = (uint32_t)tid / P;
        for (uint64_t b = ln.table_pad_from + lane_in; b < ln.table_pad_to; b += NT / P) bad |= ln.stream[b] != 0;
        for (uint64_t b = ln.ulen_pad_from + lane_in; b < ln.ulen_pad_to; b += NT / P) bad |= ln.stream[b] != 0;
    }

    // ---- decode
    Reader<NT> r;
    r.ring = &S.ring[0][tid];
    r.p = ln.payload;
    r.sw = sw;
    r.gmax = ln.payload_words ? (ln.payload_words - 1) >> 2 : 0;
    r.sh = (uint32_t)sw & (RING - 1);
    const uint16_t* lut = lut_of<NT, P>(S, k);
    const uint64_t e0 = c * a.chunk + (uint64_t)j * UNIT;  // first element of the unit
    const bool run = active && !bad;
    const uint32_t ngrp = run ? cnt >> 4 : 0u;
    // lanes of one unit keep the same group count so that the exchanges of
    // the fused outputs pair up (a unit's P lanes see the same cnt)
    uint32_t inval = 0;
    if (run && cnt) r.start(first_bit);
    for (uint32_t g = 0; g < ngrp; ++g) {
        uint32_t w[4];
        uint32_t ev[4];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if ((q & 3) == 0) r.tick();
            r.refill();
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int i = 2 * q + h;
                const uint32_t e = lookup<P>(S, lut, ln.cb, base2, r.peek(), inval);
                r.off += e & 0xFFu;
                ev[i & 3] = e;
                if ((i & 3) == 3) w[i >> 2] = syms4(ev);
            }
        }
        if constexpr (OUT == DEC_OUT_PLANES) {
            v4u v;
            v.x = w[0];
            v.y = w[1];
            v.z = w[2];
            v.w = w[3];
            *reinterpret_cast<v4u*>(ln.out + e0 + 16 * g) = v;
        } else if constexpr (OUT == DEC_OUT_U16 || OUT == DEC_OUT_U16_XOR) {
            v4u v = restore_u16(w, k);
            const uint64_t at = 2 * (e0 + 16 * g) + 16 * k;
            if constexpr (OUT == DEC_OUT_U16_XOR) v ^= *reinterpret_cast<const v4u*>(a.w0 + at);
            *reinterpret_cast<v4u*>(a.merged + at) = v;
        } else {
            const v4u v = restore_u32(w, k);
            *reinterpret_cast<v4u*>(a.merged + 4 * (e0 + 16 * g) + 16 * k) = v;
        }
    }
    if (run && cnt) {
        // the tensor's last unit: the symbols after the last full group
        const uint32_t rem = cnt & 15u;
        for (uint32_t i = 0; i < rem; ++i) {
            if ((i & 3) == 0) r.tick();
            r.refill();
            const uint32_t e = lookup<P>(S, lut, ln.cb, base2, r.peek(), inval);
            r.off += e & 0xFFu;
            const uint64_t el = e0 + 16 * ngrp + i;
            const uint8_t sym = (uint8_t)(e >> 8);
            if constexpr (OUT == DEC_OUT_PLANES) {
                ln.out[el] = sym;
            } else {
                // byte P-1-k of element el (plane k holds byte P-1-k)
                const uint64_t at = (uint64_t)P * el + (P - 1 - k);
                a.merged[at] = OUT == DEC_OUT_U16_XOR ? (uint8_t)(sym ^ a.w0[at]) : sym;
            }
        }
        r.refill();
        const uint32_t end = r.pos();
        if (inval || end != first_bit + my_bits) bad = true;
        // the unit with the chunk's last symbol: zero padding to the end of the word
        if (!bad && j == ((m_c - 1) >> 8)) {
            const uint32_t rest = (uint32_t)(32 * wc) - end;
            if (rest >= 32 || (rest && (r.peek() >> (32 - rest)) != 0)) bad = true;
        }
    }

    // ---- status, accounting, exit
    constexpr int NS = P == 1 ? 1 : P;  // streams in this workgroup
    const uint32_t slot = P == 1 ? 0u : k;
    __syncthreads();  // the ring is free again: per-stream flags and bit sums
    uint32_t* const flag = &S.ring[0][0];                                                    // [NS]
    unsigned long long* const bsum = reinterpret_cast<unsigned long long*>(&S.ring[1][0]);  // [NS]
    if (tid < NS) {
        flag[tid] = 0u;
        bsum[tid] = 0ull;
    }
    __syncthreads();
    if (bad) atomicOr(&flag[slot], 1u);
    {
        // bits of the units decoded without fault, summed per stream
        uint64_t v = (run && !bad) ? my_bits : 0u;
#pragma unroll
        for (int o = 32; o >= P; o >>= 1) v += __shfl_xor(v, o, 64);
        if ((tid & 63) < P && v) atomicAdd(&bsum[tid & 63], (unsigned long long)v);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        if (tid == q) {
            const DecStream& d = a.st[P == 1 ? sidx : (uint32_t)q];
            if (bsum[q]) atomicAdd(reinterpret_cast<unsigned long long*>(&d.ws->bits), bsum[q]);
            if (flag[q]) atomicCAS(&d.ws->status, 0, (int32_t)LECB_ERR_CORRUPT);
        }
    }
    if (tid == 0) {
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
                const uint64_t bits = __hip_atomic_load(&e.ws->bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int32_t st = __hip_atomic_load(&e.ws->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t W = e.table[a.nc - 1];
                e.res->bytes = e.header_bytes + 4 * W;
                e.res->payload_bits = bits;
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
void launch(const DecArgs& a, uint32_t wgs, hipStream_t hs) {
    hipLaunchKernelGGL((decode_kernel<NT, P, OUT>), dim3(wgs), dim3(NT), 0, hs, a);
}

}  // namespace

int launch_decode(const DecodeLaunch& L, void* stream) {
    DecArgs a{};
    const uint64_t tb = table_bytes(L.nc), ub = ulen_bytes(L.nc, L.chunk);
    const uint32_t K = units_per_chunk(L.chunk);
    a.chunk = L.chunk;
    a.log2k = (uint32_t)ilog2(K);
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
        st.ulen = reinterpret_cast<const uint16_t*>(L.stream_base[s] + tb);
        st.payload = reinterpret_cast<const uint32_t*>(L.stream_base[s] + tb + ub);
        st.payload_words = L.dev_sizes ? 0 : (L.stream_bytes[s] - tb - ub) / 4;
        st.cb = L.cb[s];
        st.header_bytes = tb + ub;
        st.stream = L.stream_base[s];
        st.table_pad_from = 4 * L.nc;
        st.table_pad_to = tb;
        st.ulen_pad_from = tb + 2 * L.nc * K;
        st.ulen_pad_to = tb + ub;
        st.out = L.out[s];
        st.res = L.res[s];
        st.ws = L.ws[s];
    }
    const uint64_t units = L.nc * K;
    const uint64_t cus = (uint64_t)device_cu_count();
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (L.out_kind == DEC_OUT_PLANES) {
        // One stream per workgroup.  Lanes per workgroup: the tables are one
        // copy per workgroup, so bigger workgroups leave more LDS for lanes
        // (2 x 1024 lanes fit a CU against 5 x 256), and fewer, bigger
        // workgroups spread evenly over the CUs.  Take the biggest size that
        // still gives every CU a workgroup (every size holds whole chunks:
        // K <= 256 units).
        const uint64_t all = units * (uint64_t)L.nstreams;
        const int nt = all >= cus * 1024 ? 1024 : all >= cus * 512 ? 512 : 256;
        a.wg_per_group = (uint32_t)((units + nt - 1) / nt);
        const uint32_t wgs = a.wg_per_group * (uint32_t)L.nstreams;
        if (nt == 1024) launch<1024, 1, DEC_OUT_PLANES>(a, wgs, hs);
        else if (nt == 512) launch<512, 1, DEC_OUT_PLANES>(a, wgs, hs);
        else launch<256, 1, DEC_OUT_PLANES>(a, wgs, hs);
    } else if (L.out_kind == DEC_OUT_U16 || L.out_kind == DEC_OUT_U16_XOR) {
        // two lanes per unit; a workgroup holds whole chunks (2K <= 512 lanes)
        if (L.nstreams != 2 || !L.merged || (L.out_kind == DEC_OUT_U16_XOR && !L.w0)) return LECB_ERR_INVALID_ARG;
        const uint64_t lanes = 2 * units;
        const int nt = lanes >= cus * 1024 ? 1024 : 512;
        const uint32_t wgs = (uint32_t)((lanes + nt - 1) / nt);
        if (L.out_kind == DEC_OUT_U16) {
            if (nt == 1024) launch<1024, 2, DEC_OUT_U16>(a, wgs, hs);
            else launch<512, 2, DEC_OUT_U16>(a, wgs, hs);
        } else {
            if (nt == 1024) launch<1024, 2, DEC_OUT_U16_XOR>(a, wgs, hs);
            else launch<512, 2, DEC_OUT_U16_XOR>(a, wgs, hs);
        }
    } else if (L.out_kind == DEC_OUT_U32) {
        // four lanes per unit; a workgroup holds whole chunks (4K lanes)
        if (L.nstreams != 4 || !L.merged) return LECB_ERR_INVALID_ARG;
        const uint64_t lanes = 4 * units;
        const int nt = 4 * K > 512 ? 1024 : 512;
        const uint32_t wgs = (uint32_t)((lanes + nt - 1) / nt);
        if (nt == 1024) launch<1024, 4, DEC_OUT_U32>(a, wgs, hs);
        else launch<512, 4, DEC_OUT_U32>(a, wgs, hs);
    } else {
        return LECB_ERR_INVALID_ARG;
    }
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

}  // namespace lecb
