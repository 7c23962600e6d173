// Huffman encode of byte symbols into stream format v2, in two launches
// (a count launch, then a pack launch).
//
// "Single-Stage Huffman Encoder for ML Compression", Methodology step 4: each
// tensor is coded directly with the codebook already resident on the device.
// "Lossless Compression for LLM Tensor Incremental Snapshots", Technical
// framework step 3 (Huffman coding of the byte groups): the plane modes read
// one byte plane straight out of the 16-bit words, and the pair mode codes
// both planes in one pass over the words (two streams, two codebooks).
//
// Work unit: a ticket of max(chunk, 16384) symbols -- G = 16384/chunk whole
// chunks, or one chunk made of chunk/16384 segments.  A segment is 256
// threads x 64 consecutive symbols.  The grid is persistent and workgroup w
// owns the contiguous tickets [w*T/W, (w+1)*T/W).  Two launches:
//   1. count_kernel: every workgroup sums the payload words of its tickets
//      (per chunk: ceil(bits / 32)) and stores that total; every thread
//      also stores the code bits of its 64 symbols;
//   2. encode_kernel: workgroup w starts at the sum of the totals of
//      workgroups 0..w-1 (the device-wide exclusive scan, done by one wave
//      per stream) and then, ticket by ticket:
//      A. each thread reads the code bits of its 64 symbols stored by the
//         count launch; a block scan gives every thread's bit offset inside
//         its chunk and every chunk's size.  With one segment per ticket the
//         thread also loads its symbols (all loads in flight at once), which
//         stay in registers for step C;
//      B. the ticket's first payload word is the running sum of the words of
//         the workgroup's earlier tickets; the chunk table entries follow;
//      C. per stream: every thread ORs its code words into an LDS image of
//         the ticket's payload (each chunk starts on a word), then the image
//         goes out with coalesced stores.  The code bits of every decode
//         unit (256 symbols = 4 threads) are the sum of its four threads'
//         bits and go out as one u16 per unit.
// No workgroup ever waits for another one.
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "lecb_internal.hpp"

namespace lecb {

namespace {

constexpr int ENC_THREADS = 256;
constexpr int ENC_WGS_PER_CU = 2;   // pack workgroups per compute unit at most (default grid)
constexpr int ENC_WGS_PER_CU_LONG = 3;   // the same for long inputs (see launch_encode)
constexpr uint64_t ENC_LONG_SEGS = 32;   // segments per workgroup that make an input long
constexpr int SPT = 64;                                  // symbols per thread in a segment
constexpr uint32_t SEG = ENC_THREADS * SPT;              // 16384
constexpr int MAX_G = SEG / LECB_MIN_CHUNK;              // chunks per ticket at most (64)
constexpr int STAGE_WORDS = SEG * 16 / 32 + MAX_G + 2;   // worst case 16 bits/symbol, + rounding + carry
// The stage holds payload word k at LDS word k + k/32.  A thread's 64 code
// words span about 64*bits/32 payload words, so with 8-bit codes the threads
// of a wave touch words 16 apart: unpadded, all 64 lanes would fall on 2 of
// the 32 banks; with the padding word every 32 they spread over all of them.
__device__ inline uint32_t st_at(uint32_t k) { return k + (k >> 5); }
constexpr int STAGE_LDS = STAGE_WORDS + STAGE_WORDS / 32 + 1;
constexpr int THREADS_PER_UNIT = LECB_UNIT_SYMBOLS / SPT;   // 4

struct StreamArgs {
    const DeviceCodebook* cb;
    uint32_t* table;
    uint16_t* ulen;                          // code bits of every decode unit
    uint32_t* payload;
    uint64_t header_bytes;
    uint64_t capacity_words;
    uint64_t table_pad_from, table_pad_to;  // byte ranges of header padding
    uint64_t ulen_pad_from, ulen_pad_to;
    uint8_t* stream;
    lecb_result* res;
    WsHeader* ws;
    uint64_t* wg_words;                      // payload words of each workgroup's tickets
};

struct EncArgs {
    const void* in;
    const void* in2;     // ENC_PAIR_XOR: symbols are the planes of in[i] ^ in2[i]
    uint64_t n;
    uint32_t chunk;
    uint32_t log2k;
    uint64_t nc;
    uint32_t G;          // chunks per ticket
    uint32_t S;          // segments per ticket
    uint64_t ntickets;
    uint32_t npack;      // pack workgroups W (ticket ranges); the count launch has F*W
    uint32_t fsplit;     // F: count workgroups per pack workgroup's range
    uint32_t* counts;    // code bits of every 64 consecutive symbols (pack_counts)
    StreamArgs st[2];
};

constexpr bool pair32_mode(int m) { return m == ENC_PAIR32_HI || m == ENC_PAIR32_LO; }
constexpr bool pair_mode(int m) { return two_stream_mode(m); }
template <int MODE> struct Streams { static constexpr int value = pair_mode(MODE) ? 2 : 1; };

__device__ inline uint32_t lo_plane(uint32_t a, uint32_t b) {
    return (a & 0xFFu) | ((a >> 8) & 0xFF00u) | ((b & 0xFFu) << 16) | ((b << 8) & 0xFF000000u);
}
__device__ inline uint32_t hi_plane(uint32_t a, uint32_t b) {
    return ((a >> 8) & 0xFFu) | ((a >> 16) & 0xFF00u) | ((b << 8) & 0xFF0000u) | (b & 0xFF000000u);
}

// The selected 16 bits of two 32-bit elements, as one word of two 16-bit values.
template <int MODE>
__device__ inline uint32_t half2(uint32_t e0, uint32_t e1) {
    if constexpr (MODE == ENC_PAIR32_HI) return (e0 >> 16) | (e1 & 0xFFFF0000u);
    else return (e0 & 0xFFFFu) | (e1 << 16);
}

// 16-bit value of element i: the word itself, its delta, or half of a 32-bit element.
template <int MODE>
__device__ inline uint32_t input_word(const EncArgs& a, uint64_t i) {
    if constexpr (pair32_mode(MODE)) {
        const uint32_t e = static_cast<const uint32_t*>(a.in)[i];
        return MODE == ENC_PAIR32_HI ? (e >> 16) : (e & 0xFFFFu);
    } else {
        uint32_t x = static_cast<const uint16_t*>(a.in)[i];
        if constexpr (MODE == ENC_PAIR_XOR) x ^= static_cast<const uint16_t*>(a.in2)[i];
        return x;
    }
}

// Symbol k of a thread's 64 (little-endian in w[16]).
__device__ inline uint32_t sym_of(const uint32_t w[16], int k) {
    return (w[k >> 2] >> (8 * (k & 3))) & 0xFFu;
}

// The thread's 64 symbols starting at i0 (nv of them below n) into w[NS][16];
// with nv == 64 all loads are issued before any is used.
template <int MODE>
__device__ inline void load64(const EncArgs& a, uint64_t i0, int nv, uint32_t w[][16]) {
    constexpr int NS = Streams<MODE>::value;
    if (nv == SPT) {
        if constexpr (MODE == ENC_BYTES) {
            const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.in) + i0);
            uint4 v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = p[q];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                w[0][4 * q] = v[q].x; w[0][4 * q + 1] = v[q].y;
                w[0][4 * q + 2] = v[q].z; w[0][4 * q + 3] = v[q].w;
            }
        } else {
            uint4 v[8];
            if constexpr (pair32_mode(MODE)) {
                const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(a.in) + i0);
                uint4 e[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) e[q] = p[q];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    v[q].x = half2<MODE>(e[2 * q].x, e[2 * q].y);
                    v[q].y = half2<MODE>(e[2 * q].z, e[2 * q].w);
                    v[q].z = half2<MODE>(e[2 * q + 1].x, e[2 * q + 1].y);
                    v[q].w = half2<MODE>(e[2 * q + 1].z, e[2 * q + 1].w);
                }
            } else {
                const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.in) + i0);
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] = p[q];
            }
            if constexpr (MODE == ENC_PAIR_XOR) {
                const uint4* p2 = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.in2) + i0);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint4 u = p2[q];
                    v[q].x ^= u.x; v[q].y ^= u.y; v[q].z ^= u.z; v[q].w ^= u.w;
                }
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if constexpr (MODE == ENC_PLANE_LO) {
                    w[0][2 * q] = lo_plane(v[q].x, v[q].y);
                    w[0][2 * q + 1] = lo_plane(v[q].z, v[q].w);
                } else {
                    w[0][2 * q] = hi_plane(v[q].x, v[q].y);
                    w[0][2 * q + 1] = hi_plane(v[q].z, v[q].w);
                }
                if constexpr (NS == 2) {
                    w[1][2 * q] = lo_plane(v[q].x, v[q].y);
                    w[1][2 * q + 1] = lo_plane(v[q].z, v[q].w);
                }
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int q = 0; q < 16; ++q) w[s][q] = 0;
        for (int k = 0; k < nv; ++k) {
            uint32_t b0, b1 = 0;
            if constexpr (MODE == ENC_BYTES) {
                b0 = static_cast<const uint8_t*>(a.in)[i0 + k];
            } else {
                const uint32_t x = input_word<MODE>(a, i0 + k);
                b0 = MODE == ENC_PLANE_LO ? (x & 0xFFu) : (x >> 8);
                b1 = x & 0xFFu;
            }
            w[0][k >> 2] |= b0 << (8 * (k & 3));
            if constexpr (NS == 2) w[1][k >> 2] |= b1 << (8 * (k & 3));
        }
    }
}

__device__ inline uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Inclusive scan of one u64 per thread over the block (two u32 counters
// packed in one u64 never carry into each other here); *total = block sum.
__device__ inline uint64_t block_inclusive_scan(uint64_t v, uint64_t* s_tmp, uint64_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_tmp[wave] = incl;
    __syncthreads();
    uint64_t before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < ENC_THREADS / 64; ++w) {
        const uint64_t x = s_tmp[w];
        if (w < wave) before += x;
        sum += x;
    }
    *total = sum;
    __syncthreads();  // s_tmp may be reused right after
    return before + incl;
}

__device__ inline void set_status(WsHeader* ws, int32_t code) {
    atomicCAS(&ws->status, 0, code);
}

struct Shared {
    uint32_t stage[STAGE_LDS];     // payload image of the ticket (one stream at a time), padded
    uint32_t enc[2][256];          // (code << 5) | len per stream
    uint8_t len[2][256];
    uint64_t incl[ENC_THREADS];    // inclusive scan of per-thread bits (stream 1 in the high half)
    uint64_t tmp[4];
    uint32_t cword[2][MAX_G];      // first payload word of each chunk, ticket-relative
    uint32_t cbits[2][MAX_G];      // bits of each chunk
    uint64_t tbase[2];
    uint64_t tbits[2];
    uint32_t twords[2];
    uint64_t run[2];               // first payload word of the next ticket
    uint32_t uncoded;
};

// The code bits of 64 consecutive symbols as the count launch stores them
// for the pack launch: stream 0 in bits 0-14, stream 1 in bits 16-30 (at
// most 64 * 16 each), bit 31 set when a valid symbol has no code word.
__device__ inline uint32_t pack_counts(uint64_t bits, bool unc) {
    return (uint32_t)(bits & 0x7FFFu) | ((uint32_t)(bits >> 32) << 16) | (unc ? 0x80000000u : 0u);
}
__device__ inline uint64_t unpack_counts(uint32_t c) {
    return (uint64_t)(c & 0x7FFFu) | ((uint64_t)((c >> 16) & 0x7FFFu) << 32);
}

// Bits of the thread's 64 symbols, per stream (nv valid); sets *unc when a
// valid symbol has no code word.
template <int NS>
__device__ inline uint64_t count_bits(const uint8_t (&len)[2][256], const uint32_t w[][16], int nv, bool* unc) {
    uint64_t packed = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        uint32_t bits = 0, mn = 16;
        if (nv == SPT) {
#pragma unroll
            for (int k = 0; k < SPT; ++k) {
                const uint32_t l = len[s][sym_of(w[s], k)];
                bits += l;
                mn = min(mn, l);
            }
        } else {
            for (int k = 0; k < nv; ++k) {
                const uint32_t l = len[s][sym_of(w[s], k)];
                bits += l;
                mn = min(mn, l);
            }
        }
        *unc |= mn == 0;
        packed |= (uint64_t)bits << (32 * s);
    }
    return packed;
}

// Pack the thread's code words into the stage at bit `pos`.  FULL: all 64
// symbols valid (else the first nv; the rest are zero bytes and get no code
// word).
//   * Code words are looked up 16 at a time (one LDS latency per 16) and
//     joined in pairs: a pair is at most 32 bits, so it enters the 64-bit
//     accumulator in one step and completes at most one word.
//   * No branches per pair.  Every pair ORs one word into the stage (which
//     is zero before packing): the completed word, or zero into the word
//     being filled.  A word shared with the neighbouring threads (the first
//     and the last) gets each thread's bits by the same OR.
template <bool FULL>
__device__ inline void pack64(Shared& S, int s, uint32_t w[16], int nv, uint32_t pos) {
    uint32_t widx = pos >> 5;
    uint32_t used = pos & 31u;
    uint64_t acc = 0;
    // 16 symbols per round; the symbol words move down by 4 after each round
    // (w is used up), so every index stays a constant without unrolling all
    // 64 symbols
    uint32_t* const ww = w;
#pragma unroll 1
    for (int g = 0; g < SPT / 16; ++g) {
        uint32_t e[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t x = S.enc[s][sym_of(ww, i)];
            e[i] = (FULL || 16 * g + i < nv) ? x : 0u;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t e0 = e[2 * q], e1 = e[2 * q + 1];
            const uint32_t l0 = e0 & 31u, l1 = e1 & 31u;
            const uint32_t c2 = ((e0 >> 5) << l1) | (e1 >> 5);  // at most 32 bits
            used += l0 + l1;
            acc |= (uint64_t)c2 << ((64 - used) & 63);  // ends at bit `used` from the top
            const uint32_t full = used >> 5;             // used <= 63
            atomicOr(&S.stage[st_at(widx)], (uint32_t)(acc >> 32) & (0u - full));
            acc <<= 32 * full;
            widx += full;
            used &= 31u;
        }
#pragma unroll
        for (int i = 0; i < 12; ++i) ww[i] = ww[i + 4];
    }
    if (used) atomicOr(&S.stage[st_at(widx)], (uint32_t)(acc >> 32));
}

// Code bits of the decode unit of the thread (the 4 threads of a unit are
// consecutive lanes of a wave); every lane receives its unit's total.
__device__ inline uint32_t unit_bits(uint32_t mine) {
    uint32_t v = mine + __shfl_xor(mine, 1, 64);
    return v + __shfl_xor(v, 2, 64);
}

// First ticket of workgroup w when T tickets are split over W workgroups.
__device__ inline uint64_t first_ticket(uint64_t w, uint64_t T, uint64_t W) { return w * T / W; }

// Bits of each chunk of ticket `tk` (per stream, lanes 0..nch-1 of wave s
// receive chunk `lane`'s bits); w keeps the symbols when the ticket is one
// segment, and incl/tmp/len are the caller's LDS.  STORED: the bits come
// from the count launch's per-thread totals (the symbols are loaded only
// when the ticket is one segment); otherwise they are summed here from the
// symbols and stored for the pack launch.
template <int MODE, bool STORED>
__device__ inline void ticket_bits(const EncArgs& a, uint64_t tk, const uint8_t (&len)[2][256],
                                   uint64_t* incl_lds, uint64_t* tmp, uint32_t w[][16], bool* unc,
                                   uint32_t* nch_out, uint32_t* nseg_out, uint64_t* chunk_acc) {
    constexpr int NS = Streams<MODE>::value;
    const int tid = threadIdx.x;
    const uint64_t c0 = tk * a.G;
    const uint32_t nch = (uint32_t)min<uint64_t>(a.G, a.nc - c0);
    const uint64_t tbeg = c0 * a.chunk;
    const uint64_t tend = min(tbeg + (uint64_t)a.G * a.chunk, a.n);
    const uint32_t nseg = (uint32_t)((tend - tbeg + SEG - 1) / SEG);
    uint64_t acc = 0;
    for (uint32_t g = 0; g < nseg; ++g) {
        const uint64_t i0 = tbeg + (uint64_t)g * SEG + (uint64_t)tid * SPT;
        const int nv = i0 >= tend ? 0 : (int)min<uint64_t>(SPT, tend - i0);
        uint64_t bits;
        if constexpr (STORED) {
            const uint32_t c = nv > 0 ? a.counts[i0 / SPT] : 0u;
            if (nseg == 1) load64<MODE>(a, i0, nv, w);
            bits = unpack_counts(c);
            *unc |= (c >> 31) != 0;
        } else {
            load64<MODE>(a, i0, nv, w);
            bool u = false;
            bits = count_bits<NS>(len, w, nv, &u);
            *unc |= u;
            if (nv > 0) a.counts[i0 / SPT] = pack_counts(bits, u);
        }
        uint64_t total;
        const uint64_t incl = block_inclusive_scan(bits, tmp, &total);
        if (nseg == 1) incl_lds[tid] = incl;
        acc += total;
    }
    *nch_out = nch;
    *nseg_out = nseg;
    *chunk_acc = acc;
}

// Bits of chunk `lane` of the ticket for stream s (0 for lanes >= nch).
__device__ inline uint32_t chunk_bits_of(const uint64_t* incl_lds, int lane, int s, uint32_t nch,
                                         uint32_t nseg, uint32_t L, uint64_t chunk_acc) {
    if (nseg == 1) {
        if (lane >= (int)nch) return 0;
        const uint64_t hi = incl_lds[(lane + 1) * L - 1];
        const uint64_t lo = lane ? incl_lds[lane * L - 1] : 0ull;
        return (uint32_t)((hi - lo) >> (32 * s));
    }
    return lane == 0 ? (uint32_t)(chunk_acc >> (32 * s)) : 0u;
}

// Launch 1: payload words of every workgroup's tickets, per stream.  Each
// pack workgroup's ticket range is counted by F workgroups (more loads in
// flight than one workgroup walking it), whose totals follow each other.
template <int MODE>
__global__ __launch_bounds__(ENC_THREADS) void count_kernel(EncArgs a) {
    constexpr int NS = Streams<MODE>::value;
    __shared__ uint8_t len[2][256];
    __shared__ uint64_t incl[ENC_THREADS];
    __shared__ uint64_t tmp[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int s = 0; s < NS; ++s) len[s][tid] = (uint8_t)(a.st[s].cb->enc[tid] & 31u);
    __syncthreads();
    const uint32_t L = a.chunk >= SEG ? ENC_THREADS : a.chunk / SPT;
    // the range of pack workgroup w = blockIdx / F, split F ways
    const uint64_t pw = blockIdx.x / a.fsplit, f = blockIdx.x % a.fsplit;
    const uint64_t r0 = first_ticket(pw, a.ntickets, a.npack), r1 = first_ticket(pw + 1, a.ntickets, a.npack);
    const uint64_t t0 = r0 + (r1 - r0) * f / a.fsplit, t1 = r0 + (r1 - r0) * (f + 1) / a.fsplit;
    uint64_t words = 0;  // wave s, stream s
    for (uint64_t tk = t0; tk < t1; ++tk) {
        uint32_t w[NS][16];
        bool unc = false;
        uint32_t nch, nseg;
        uint64_t acc;
        ticket_bits<MODE, false>(a, tk, len, incl, tmp, w, &unc, &nch, &nseg, &acc);
        __syncthreads();
        if (wave < NS) {
            const uint32_t cb = chunk_bits_of(incl, lane, wave, nch, nseg, L, acc);
            words += wave_sum_u64((cb + 31) >> 5);
        }
        __syncthreads();
    }
    if (wave < NS && lane == 0) a.st[wave].wg_words[blockIdx.x] = words;
}

// Launch 2: pack (see the top of the file).  A 256-lane workgroup is one
// wave per SIMD, so ENC_WGS_PER_CU workgroups per CU are as many waves per
// SIMD: the second launch bound (minimum waves per SIMD) allows registers for
// that many.
template <int MODE>
__global__ __launch_bounds__(ENC_THREADS, ENC_WGS_PER_CU) void encode_kernel(EncArgs a) {
    constexpr int NS = Streams<MODE>::value;
    __shared__ Shared S;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const uint32_t e = a.st[s].cb->enc[tid];
        S.enc[s][tid] = e;
        S.len[s][tid] = (uint8_t)(e & 31u);
    }
    // first payload word of this workgroup: the words of workgroups 0..w-1,
    // summed by all threads (independent loads, one latency)
    {
        uint64_t part[2] = {0, 0};
#pragma unroll 4
        for (uint32_t v = tid; v < blockIdx.x * a.fsplit; v += ENC_THREADS) {
#pragma unroll
            for (int s = 0; s < NS; ++s) part[s] += a.st[s].wg_words[v];
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const uint64_t x = wave_sum_u64(part[s]);
            if (lane == 0) S.incl[NS * wave + s] = x;
        }
    }
    if (tid == 0) S.uncoded = 0;
    __syncthreads();
    if (tid < NS) {
        uint64_t sum = 0;
        for (int v = 0; v < ENC_THREADS / 64; ++v) sum += S.incl[NS * v + tid];
        S.run[tid] = sum;
    }
    __syncthreads();
    const uint32_t K = 1u << a.log2k;
    const uint32_t L = a.chunk >= SEG ? ENC_THREADS : a.chunk / SPT;  // threads per chunk in a segment
    const uint64_t t0 = first_ticket(blockIdx.x, a.ntickets, gridDim.x);
    const uint64_t t1 = first_ticket(blockIdx.x + 1ull, a.ntickets, gridDim.x);

    for (uint64_t T = t0; T < t1; ++T) {
        const uint64_t c0 = T * a.G;                                   // first chunk
        const uint64_t tbeg = c0 * a.chunk;                            // first symbol
        const uint64_t tend = min(tbeg + (uint64_t)a.G * a.chunk, a.n);

        // ---- A: bits of every chunk of the ticket
        uint32_t w[NS][16];
        bool unc = false;
        uint32_t nch, nseg;
        uint64_t chunk_bits_acc;  // nseg > 1: the one chunk's bits (packed per stream)
        ticket_bits<MODE, true>(a, T, S.len, S.incl, S.tmp, w, &unc, &nch, &nseg, &chunk_bits_acc);
        if (unc) atomicOr(&S.uncoded, 1u);
        __syncthreads();
        // ---- B: chunk sizes, word offsets and the ticket's place in the
        // payload (wave s handles stream s)
        if (wave < NS) {
            const int s = wave;
            const StreamArgs& sa = a.st[s];
            const uint32_t cb = chunk_bits_of(S.incl, lane, s, nch, nseg, L, chunk_bits_acc);
            const uint32_t cw = (cb + 31) >> 5;
            uint32_t incl = cw;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t t = __shfl_up(incl, o, 64);
                if (lane >= o) incl += t;
            }
            if (lane < (int)nch) {
                S.cword[s][lane] = incl - cw;
                S.cbits[s][lane] = cb;
            }
            const uint32_t tw = __shfl(incl, 63, 64);
            const uint64_t tbits = wave_sum_u64(cb);
            const uint64_t base = S.run[s];
            if (lane < (int)nch) sa.table[c0 + lane] = (uint32_t)(base + incl);
            if (lane == 0) {
                S.twords[s] = tw;
                S.tbase[s] = base;
                S.run[s] = base + tw;
                atomicAdd(reinterpret_cast<unsigned long long*>(&sa.ws->bits), (unsigned long long)tbits);
                if (T == a.ntickets - 1)
                    __hip_atomic_store(&sa.ws->words, base + tw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (S.uncoded) set_status(sa.ws, LECB_ERR_UNCODED_SYMBOL);
                if (base + tw >= (1ull << 32)) set_status(sa.ws, LECB_ERR_TOO_LARGE);
                else if (base + tw > sa.capacity_words) set_status(sa.ws, LECB_ERR_CAPACITY);
            }
        }
        __syncthreads();

        // ---- C: pack, segment by segment (the symbols of a segment are loaded
        // once for both streams), stream by stream
        uint32_t TB[NS];      // S > 1: chunk-relative bit offset of the segment
        uint32_t carry[NS];   // S > 1: partial last word of the previous segment
#pragma unroll
        for (int s = 0; s < NS; ++s) TB[s] = carry[s] = 0;
        for (uint32_t g = 0; g < nseg; ++g) {
            const uint64_t i0 = tbeg + (uint64_t)g * SEG + (uint64_t)tid * SPT;
            const int nv = i0 >= tend ? 0 : (int)min<uint64_t>(SPT, tend - i0);
            uint64_t incl, own, seg_total = 0;
            if (nseg == 1) {
                incl = S.incl[tid];
                own = incl - (tid ? S.incl[tid - 1] : 0ull);
            } else {
                // the segment's scan again (step A kept only totals)
                const uint32_t c = nv > 0 ? a.counts[i0 / SPT] : 0u;
                load64<MODE>(a, i0, nv, w);
                own = unpack_counts(c);
                incl = block_inclusive_scan(own, S.tmp, &seg_total);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const StreamArgs& st = a.st[s];
                const uint32_t twords = S.twords[s];
                const uint32_t mine = (uint32_t)(own >> (32 * s));  // this thread's bits
                uint32_t pos, ch;
                uint32_t r0 = 0, w0 = 0, touched;
                if (nseg == 1) {
                    ch = tid / L;
                    const uint64_t before = ch ? S.incl[ch * L - 1] : 0ull;
                    const uint32_t ts = (uint32_t)((incl - before) >> (32 * s)) - mine;  // chunk-relative start bit
                    pos = (ch < nch ? S.cword[s][ch] * 32u : 0u) + ts;
                    touched = twords;
                    for (uint32_t k = tid; k < touched; k += ENC_THREADS) S.stage[st_at(k)] = 0u;
                } else {
                    ch = 0;
                    const uint32_t seg_bits = (uint32_t)(seg_total >> (32 * s));
                    const uint32_t excl = (uint32_t)(incl >> (32 * s)) - mine;
                    r0 = TB[s] & 31u;
                    w0 = TB[s] >> 5;
                    pos = r0 + excl;
                    touched = (r0 + seg_bits + 31) >> 5;
                    for (uint32_t k = tid; k <= touched; k += ENC_THREADS) S.stage[st_at(k)] = k ? 0u : carry[s];
                    TB[s] += seg_bits;
                }
                // the unit's code bits: unit u of the ticket's chunk ch (units
                // past n hold no symbols and get 0)
                {
                    const uint32_t ub = unit_bits(mine);
                    const uint64_t u = nseg == 1
                                           ? (c0 + ch) * K + (tid % L) / THREADS_PER_UNIT
                                           : c0 * K + (uint64_t)g * (SEG / LECB_UNIT_SYMBOLS) + tid / THREADS_PER_UNIT;
                    if ((tid & (THREADS_PER_UNIT - 1)) == 0 && ch < nch) st.ulen[u] = (uint16_t)ub;
                }
                __syncthreads();
                if (nv == SPT && ch < nch)
                    pack64<true>(S, s, w[s], nv, pos);
                else if (nv > 0 && ch < nch)
                    pack64<false>(S, s, w[s], nv, pos);
                __syncthreads();  // stage complete
                const uint64_t tbase = S.tbase[s];
                const bool write_ok = tbase + twords <= st.capacity_words && !S.uncoded;
                if (nseg == 1) {
                    if (write_ok) {
                        uint32_t* dst = st.payload + tbase;
                        uint32_t k = tid;
                        for (; k + 3 * ENC_THREADS < twords; k += 4 * ENC_THREADS) {
                            uint32_t v[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q) v[q] = S.stage[st_at(k + q * ENC_THREADS)];
#pragma unroll
                            for (int q = 0; q < 4; ++q) dst[k + q * ENC_THREADS] = v[q];
                        }
                        for (; k < twords; k += ENC_THREADS) dst[k] = S.stage[st_at(k)];
                    }
                } else {
                    const bool last_seg = g + 1 == nseg;
                    const uint32_t full = TB[s] / 32 - w0;  // words completed by this segment
                    const uint32_t nwrite = last_seg ? touched : full;
                    if (write_ok) {
                        uint32_t* dst = st.payload + tbase + w0;
                        for (uint32_t k = tid; k < nwrite; k += ENC_THREADS) dst[k] = S.stage[st_at(k)];
                    }
                    carry[s] = S.stage[st_at(full)];
                }
                __syncthreads();
            }
        }
        // a short last chunk of a chunk size above SEG: its units past the
        // last segment hold no symbols
        if (a.chunk > SEG && nseg * (SEG / LECB_UNIT_SYMBOLS) < K) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                for (uint32_t u = nseg * (SEG / LECB_UNIT_SYMBOLS) + tid; u < K; u += ENC_THREADS)
                    a.st[s].ulen[c0 * K + u] = 0;
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const StreamArgs& st = a.st[s];
            if (c0 + nch == a.nc) {
                for (uint64_t b = st.table_pad_from + tid; b < st.table_pad_to; b += ENC_THREADS)
                    st.stream[b] = 0;
                for (uint64_t b = st.ulen_pad_from + tid; b < st.ulen_pad_to; b += ENC_THREADS)
                    st.stream[b] = 0;
            }
        }
        __syncthreads();
    }

    // ---- exit: the last workgroup publishes the results and resets the workspace
    if (tid == 0) {
        __threadfence();
        WsHeader* ws0 = a.st[0].ws;
        const uint32_t done = __hip_atomic_fetch_add(&ws0->exit_count, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                WsHeader* ws = a.st[s].ws;
                const uint64_t words = __hip_atomic_load(&ws->words, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t bits = __hip_atomic_load(&ws->bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int32_t stt = __hip_atomic_load(&ws->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                a.st[s].res->bytes = a.st[s].header_bytes + 4 * words;
                a.st[s].res->payload_bits = bits;
                a.st[s].res->status = stt;
                a.st[s].res->reserved = 0;
                ws->words = 0;
                ws->bits = 0;
                ws->status = 0;
            }
            __threadfence();
            __hip_atomic_store(&ws0->exit_count, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

namespace {

// Calls f(std::integral_constant<int, mode>) for a valid mode.
template <typename F>
hipError_t with_mode(int mode, F&& f) {
    switch (mode) {
        case ENC_BYTES: return f(std::integral_constant<int, ENC_BYTES>{});
        case ENC_PLANE_LO: return f(std::integral_constant<int, ENC_PLANE_LO>{});
        case ENC_PLANE_HI: return f(std::integral_constant<int, ENC_PLANE_HI>{});
        case ENC_PAIR: return f(std::integral_constant<int, ENC_PAIR>{});
        case ENC_PAIR_XOR: return f(std::integral_constant<int, ENC_PAIR_XOR>{});
        case ENC_PAIR32_HI: return f(std::integral_constant<int, ENC_PAIR32_HI>{});
        case ENC_PAIR32_LO: return f(std::integral_constant<int, ENC_PAIR32_LO>{});
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int launch_encode(const EncodeLaunch& L, void* stream) {
    EncArgs a{};
    a.in = L.in;
    a.in2 = L.in2;
    a.n = L.n;
    a.chunk = L.chunk;
    a.log2k = (uint32_t)ilog2(units_per_chunk(L.chunk));
    a.nc = L.nc;
    a.counts = L.counts;
    if (!a.counts) return LECB_ERR_INVALID_ARG;
    a.G = L.chunk >= SEG ? 1u : SEG / L.chunk;
    a.S = L.chunk > SEG ? L.chunk / SEG : 1u;
    a.ntickets = (L.nc + a.G - 1) / a.G;
    const int ns = pair_mode(L.mode) ? 2 : 1;
    for (int s = 0; s < ns; ++s)
        if (!L.st[s].cb || !L.st[s].out || !L.st[s].res || !L.st[s].ws) return LECB_ERR_INVALID_ARG;
    const uint64_t tb = table_bytes(L.nc), ub = ulen_bytes(L.nc, L.chunk);
    for (int s = 0; s < ns; ++s) {
        StreamArgs& st = a.st[s];
        st.cb = L.st[s].cb;
        st.stream = L.st[s].out;
        st.table = reinterpret_cast<uint32_t*>(L.st[s].out);
        st.ulen = reinterpret_cast<uint16_t*>(L.st[s].out + tb);
        st.payload = reinterpret_cast<uint32_t*>(L.st[s].out + tb + ub);
        st.header_bytes = tb + ub;
        st.capacity_words = (L.st[s].capacity - (tb + ub)) / 4;
        st.table_pad_from = 4 * L.nc;
        st.table_pad_to = tb;
        st.ulen_pad_from = tb + 2 * L.nc * units_per_chunk(L.chunk);
        st.ulen_pad_to = tb + ub;
        st.res = L.st[s].res;
        st.ws = L.st[s].ws;
        st.wg_words = reinterpret_cast<uint64_t*>(L.st[s].ws + 1);  // room for nc >= grid values
    }
    // Both launches split the tickets over the same workgroups (static
    // ranges; no workgroup waits for another).  By default the grid is the
    // number of pack workgroups that fit on all compute units together, at
    // most ENC_WGS_PER_CU per unit: measured on 32 Mi int8 symbols, byte-mode
    // pack workgroups at 2 per CU took 70 us against 89 at 3 and 108 at 4 (the
    // ones that fit), and the two-plane mode is fastest at the 2 that fit.
    // Long inputs (at least ENC_LONG_SEGS segments per workgroup at that
    // grid) take 3 per CU, even where only 2 fit: the finer ticket ranges
    // even out the workgroups' ends (512 Mi 16-bit words in 65536-symbol
    // chunks: 0.99 ms against 1.09; 4 GiB of bytes: no change, ~4.9 ms).
    uint64_t grid_wgs = L.grid;
    if (L.mode < 0 || L.mode >= ENC_NUM_MODES) return LECB_ERR_INVALID_ARG;
    if (grid_wgs == 0) {
        // resident pack workgroups per CU, asked of the runtime once per
        // (device, mode); concurrent first calls store the same value
        static std::atomic<int> per_cu[MAX_DEVICES][ENC_NUM_MODES];
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return LECB_ERR_HIP;
        int pc = per_cu[dev][L.mode].load(std::memory_order_relaxed);
        if (pc == 0) {
            int nb = 0;
            const hipError_t e = with_mode(L.mode, [&](auto m) {
                return hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, encode_kernel<decltype(m)::value>,
                                                                    ENC_THREADS, 0);
            });
            if (e != hipSuccess || nb < 1) return LECB_ERR_HIP;
            pc = nb < ENC_WGS_PER_CU ? nb : ENC_WGS_PER_CU;
            per_cu[dev][L.mode].store(pc, std::memory_order_relaxed);
        }
        const uint64_t cus = (uint64_t)device_cu_count();
        grid_wgs = cus * pc;
        if (a.ntickets * a.S >= ENC_LONG_SEGS * grid_wgs) grid_wgs = cus * ENC_WGS_PER_CU_LONG;
    }
    const uint64_t nwg = grid_wgs < a.ntickets ? grid_wgs : a.ntickets;
    const dim3 grid((uint32_t)nwg), block(ENC_THREADS);
    // the workspace holds one total per chunk: F * W of them must fit
    a.npack = (uint32_t)nwg;
    a.fsplit = 4 * nwg <= a.nc ? 4u : 1u;
    const dim3 cgrid((uint32_t)(nwg * a.fsplit));
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    with_mode(L.mode, [&](auto m) {
        constexpr int M = decltype(m)::value;
        hipLaunchKernelGGL(count_kernel<M>, cgrid, block, 0, hs, a);
        hipLaunchKernelGGL(encode_kernel<M>, grid, block, 0, hs, a);
        return hipSuccess;
    });
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

}  // namespace lecb
