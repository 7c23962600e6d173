// Huffman encode of byte symbols into stream format v1, in ONE launch.
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
// threads x 64 consecutive symbols.  One 256-thread workgroup owns one ticket
// at a time (persistent grid; tickets come from an atomic counter, so every
// ticket a workgroup waits on is owned by a running workgroup).  Per ticket:
//   A. each thread loads its 64 symbols (all loads in flight at once) and
//      sums their code lengths; a block scan gives every thread's bit offset
//      inside its chunk and every chunk's size.  With one segment per ticket
//      the symbols stay in registers for step C;
//   B. per stream, the ticket's word count is published at once; decoupled
//      look-back over the tickets before it -> the ticket's first payload
//      word.  Flags are 64-bit {epoch tag, state, value}, so no call ever
//      clears them; the look-back waits only on the tickets nearer than the
//      nearest published inclusive prefix, and it runs after the first
//      packing below, when those are mostly published;
//   C. per stream: every thread ORs its code words into an LDS image of the
//      ticket's payload (each chunk starts on a word), then the image goes
//      out with coalesced stores.  While packing, a thread whose bit range
//      holds the start s_j of a decode unit records that unit's gap: the
//      distance from s_j to the first code word that starts at or after it.
#include <hip/hip_runtime.h>

#include "lecb_internal.hpp"

namespace lecb {

namespace {

constexpr int ENC_THREADS = 256;
constexpr int SPT = 64;                                  // symbols per thread in a segment
constexpr uint32_t SEG = ENC_THREADS * SPT;              // 16384
constexpr int MAX_G = SEG / LECB_MIN_CHUNK;              // chunks per ticket at most (64)
constexpr int STAGE_WORDS = SEG * 16 / 32 + MAX_G + 2;   // worst case 16 bits/symbol, + rounding + carry
constexpr int MAX_K = LECB_MAX_CHUNK / LECB_UNIT_SYMBOLS; // units per chunk at most (256)
constexpr uint64_t FLAG_VALUE_MASK = (1ull << 34) - 1;
constexpr uint32_t ST_AGG = 1, ST_PREFIX = 2;
constexpr uint32_t NO_BOUNDARY = 0xFFFFFFFFu;

struct StreamArgs {
    const DeviceCodebook* cb;
    uint32_t* table;
    uint8_t* gaps;
    uint32_t* payload;
    uint64_t header_bytes;
    uint64_t capacity_words;
    uint64_t table_pad_from, table_pad_to;  // byte ranges of header padding
    uint64_t gap_pad_from, gap_pad_to;
    uint8_t* stream;
    lecb_result* res;
    WsHeader* ws;
    uint64_t* flags;                         // one per ticket
};

struct EncArgs {
    const void* in;
    uint64_t n;
    uint32_t chunk;
    uint32_t log2k;
    uint64_t nc;
    uint32_t G;          // chunks per ticket
    uint32_t S;          // segments per ticket
    uint64_t ntickets;
    StreamArgs st[2];
};

template <int MODE> struct Streams { static constexpr int value = MODE == ENC_PAIR ? 2 : 1; };

__device__ inline uint32_t lo_plane(uint32_t a, uint32_t b) {
    return (a & 0xFFu) | ((a >> 8) & 0xFF00u) | ((b & 0xFFu) << 16) | ((b << 8) & 0xFF000000u);
}
__device__ inline uint32_t hi_plane(uint32_t a, uint32_t b) {
    return ((a >> 8) & 0xFFu) | ((a >> 16) & 0xFF00u) | ((b << 8) & 0xFF0000u) | (b & 0xFF000000u);
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
            const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.in) + i0);
            uint4 v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = p[q];
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
                const uint32_t x = static_cast<const uint16_t*>(a.in)[i0 + k];
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

__device__ inline uint64_t make_flag(uint32_t tag, uint32_t state, uint64_t value) {
    return ((uint64_t)tag << 36) | ((uint64_t)state << 34) | (value & FLAG_VALUE_MASK);
}

// Bound on polling rounds while waiting for a predecessor's flag.  Owners of
// earlier tickets publish within microseconds; only a workspace that was not
// zero-filled (stale ticket counter) could leave a flag unpublished, and then
// the call gives up with status WORKSPACE instead of waiting forever.
constexpr uint32_t SPIN_LIMIT = 1u << 24;

constexpr int LB_SLOTS = 4;  // tickets each lane watches per round: 256 per round

// Exclusive prefix (in payload words) of ticket c; run by the 64 lanes of one
// wave.  A round covers the 256 tickets below `end`: slot i of lane l watches
// ticket end-1-(64*i+l), so offset 64*i+l counts outwards from the nearest.
// The round is complete once every ticket nearer than the nearest inclusive
// prefix (state PREFIX) in it is published; then their values and that prefix
// are added up.  With no prefix in the round all 256 aggregates are added and
// the window moves down.  *timed_out is set when SPIN_LIMIT was reached.
__device__ uint64_t look_back(uint64_t* flags, int64_t c, uint32_t tag, bool* timed_out) {
    const int lane = threadIdx.x & 63;
    uint64_t excl = 0;
    int64_t end = c;
    uint32_t spins = 0;
    while (end > 0) {
        uint64_t f[LB_SLOTS];
        bool have[LB_SLOTS];
#pragma unroll
        for (int i = 0; i < LB_SLOTS; ++i) {
            f[i] = make_flag(tag, ST_PREFIX, 0);  // before ticket 0: prefix 0
            have[i] = end - 1 - (64 * i + lane) < 0;
        }
        int stop;  // offset of the nearest prefix, or 64*LB_SLOTS when none
        for (;;) {
#pragma unroll
            for (int i = 0; i < LB_SLOTS; ++i) {
                if (!have[i]) {
                    f[i] = __hip_atomic_load(&flags[end - 1 - (64 * i + lane)], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
                    have[i] = (uint32_t)(f[i] >> 36) == tag && ((f[i] >> 34) & 3u) != 0;
                }
            }
            // every slot nearer than the nearest prefix (and that prefix) must be published
            bool ok = true;
            stop = 64 * LB_SLOTS;
#pragma unroll
            for (int i = 0; i < LB_SLOTS; ++i) {
                if (stop == 64 * LB_SLOTS) {
                    const uint64_t pm = __ballot(have[i] && ((f[i] >> 34) & 3u) == ST_PREFIX);
                    const uint64_t vm = __ballot(have[i]);
                    const uint64_t need = pm ? (pm ^ (pm - 1)) : ~0ull;
                    ok = ok && (vm & need) == need;
                    if (pm) stop = 64 * i + (int)__builtin_ctzll(pm);
                }
            }
            if (ok) break;
            if (++spins >= SPIN_LIMIT) {
                *timed_out = true;
                return excl;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        uint64_t part = 0;
#pragma unroll
        for (int i = 0; i < LB_SLOTS; ++i)
            if (64 * i + lane <= stop) part += f[i] & FLAG_VALUE_MASK;
        excl += wave_sum_u64(part);
        if (stop < 64 * LB_SLOTS) break;
        end -= 64 * LB_SLOTS;
    }
    return excl;
}

__device__ inline void set_status(WsHeader* ws, int32_t code) {
    atomicCAS(&ws->status, 0, code);
}

struct Shared {
    uint32_t stage[STAGE_WORDS];   // payload image of the ticket (one stream at a time)
    uint32_t enc[2][256];          // (code << 5) | len per stream
    uint8_t len[2][256];
    uint64_t incl[ENC_THREADS];    // inclusive scan of per-thread bits (stream 1 in the high half)
    uint64_t tmp[4];
    uint32_t cword[2][MAX_G];      // first payload word of each chunk, ticket-relative
    uint32_t cbits[2][MAX_G];      // bits of each chunk
    uint8_t gap[2][MAX_K];         // unit gaps of the ticket's chunks (G*K <= MAX_K)
    uint64_t tbase[2];
    uint64_t tbits[2];
    uint32_t twords[2];
    uint32_t ticket;
    uint32_t tag;
    uint32_t uncoded;
};

// Bits of the thread's 64 symbols, per stream (nv valid); sets *unc when a
// valid symbol has no code word.
template <int NS>
__device__ inline uint64_t count_bits(const Shared& S, const uint32_t w[][16], int nv, bool* unc) {
    uint64_t packed = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        uint32_t bits = 0, mn = 16;
        if (nv == SPT) {
#pragma unroll
            for (int k = 0; k < SPT; ++k) {
                const uint32_t l = S.len[s][sym_of(w[s], k)];
                bits += l;
                mn = min(mn, l);
            }
        } else {
            for (int k = 0; k < nv; ++k) {
                const uint32_t l = S.len[s][sym_of(w[s], k)];
                bits += l;
                mn = min(mn, l);
            }
        }
        *unc |= mn == 0;
        packed |= (uint64_t)bits << (32 * s);
    }
    return packed;
}

// Record the gaps of all unit starts s_j in (prev, p]: their first code-word
// start at or after them is p.  j/nb: the next unit start and its index.
__device__ inline void gaps_upto(uint32_t p, uint32_t& j, uint32_t& nb, uint32_t wc, uint32_t K,
                                 uint32_t log2k, uint8_t* gap) {
    while (nb <= p) {
        gap[j] = (uint8_t)(p - nb);
        ++j;
        nb = j < K ? (uint32_t)(((uint64_t)j * wc) >> log2k) << 5 : NO_BOUNDARY;
    }
}

// Pack the thread's code words into the stage at bit `pos` and record the
// gaps of the unit starts in its chunk-relative bit range [ts, ...).  FULL:
// all 64 symbols valid (else the first nv).
template <bool FULL>
__device__ inline void pack64(Shared& S, int s, const uint32_t w[16], int nv, uint32_t pos,
                              uint32_t ts, uint32_t wc, uint32_t K, uint32_t log2k, uint8_t* gap) {
    // first unit start at or after ts: s_j = 32*floor(j*wc/K) >= ts
    uint32_t j = wc ? (uint32_t)((((uint64_t)((ts + 31) >> 5)) * K + wc - 1) / wc) : K;
    uint32_t nb = j < K ? (uint32_t)(((uint64_t)j * wc) >> log2k) << 5 : NO_BOUNDARY;
    uint32_t p = ts;  // chunk-relative start of the next code word
    uint32_t widx = pos >> 5;
    uint32_t used = pos & 31u;
    uint64_t acc = 0;
    gaps_upto(p, j, nb, wc, K, log2k, gap);  // a unit starting exactly at ts
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        const uint32_t e = (FULL || k < nv) ? S.enc[s][sym_of(w, k)] : 0u;
        const uint32_t len = e & 31u;
        const uint32_t pk = p;  // start of code word k
        p += len;
        used += len;
        acc |= (uint64_t)(e >> 5) << ((64 - used) & 63);  // ends at bit `used` from the top
        if (k & 1) {
            // unit starts in (start of word k-1, start of word k+1]: checked once
            // per pair; the one after the start of word k-1 but at or before pk
            // gets pk, the rest (up to p) get p
            if (p >= nb) {
                gaps_upto(pk, j, nb, wc, K, log2k, gap);
                if (k + 1 < SPT) gaps_upto(p, j, nb, wc, K, log2k, gap);
            }
            // OR the word being filled (idempotent while it grows), move on once full
            atomicOr(&S.stage[widx], (uint32_t)(acc >> 32));
            const bool full = used >= 32;
            acc = full ? acc << 32 : acc;
            widx += full ? 1u : 0u;
            used &= 31u;
        }
    }
    if (used) atomicOr(&S.stage[widx], (uint32_t)(acc >> 32));
    // unit starts after the last code word's start but before the range end:
    // their first boundary is the end of this thread's range (= p)
    while (nb < p) {
        gap[j] = (uint8_t)(p - nb);
        ++j;
        nb = j < K ? (uint32_t)(((uint64_t)j * wc) >> log2k) << 5 : NO_BOUNDARY;
    }
}

template <int MODE>
__global__ __launch_bounds__(ENC_THREADS, MODE == ENC_PAIR ? 2 : 4) void encode_kernel(EncArgs a) {
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
    if (tid == 0) {
        const uint32_t e = __hip_atomic_load(&a.st[0].ws->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        S.tag = (e % 0x0FFFFFFFu) + 1;
    }
    __syncthreads();
    const uint32_t tag = S.tag;
    const uint32_t K = 1u << a.log2k;
    const uint32_t L = a.chunk >= SEG ? ENC_THREADS : a.chunk / SPT;  // threads per chunk in a segment

    for (;;) {
        if (tid == 0) {
            S.ticket = atomicAdd(&a.st[0].ws->ticket, 1u);
            S.uncoded = 0;
        }
        __syncthreads();
        const uint64_t T = S.ticket;
        if (T >= a.ntickets) break;

        const uint64_t c0 = T * a.G;                                   // first chunk
        const uint32_t nch = (uint32_t)min<uint64_t>(a.G, a.nc - c0);   // chunks in the ticket
        const uint64_t tbeg = c0 * a.chunk;                            // first symbol
        const uint64_t tend = min(tbeg + (uint64_t)a.G * a.chunk, a.n);
        const uint32_t nseg = (uint32_t)((tend - tbeg + SEG - 1) / SEG);

        // ---- A: bits of every chunk of the ticket
        uint32_t w[NS][16];
        bool unc = false;
        uint64_t chunk_bits_acc = 0;  // S > 1: the one chunk's bits so far (packed per stream)
        for (uint32_t g = 0; g < nseg; ++g) {
            const uint64_t i0 = tbeg + (uint64_t)g * SEG + (uint64_t)tid * SPT;
            const int nv = i0 >= tend ? 0 : (int)min<uint64_t>(SPT, tend - i0);
            load64<MODE>(a, i0, nv, w);
            const uint64_t bits = count_bits<NS>(S, w, nv, &unc);
            uint64_t total;
            const uint64_t incl = block_inclusive_scan(bits, S.tmp, &total);
            if (nseg == 1) S.incl[tid] = incl;
            chunk_bits_acc += total;
        }
        if (unc) atomicOr(&S.uncoded, 1u);
        __syncthreads();
        // chunk sizes and ticket-relative word offsets: wave s handles stream s
        if (wave < NS) {
            const int s = wave;
            uint32_t cb = 0;
            if (nseg == 1) {
                if (lane < (int)nch) {
                    const uint64_t hi = S.incl[(lane + 1) * L - 1];
                    const uint64_t lo = lane ? S.incl[lane * L - 1] : 0ull;
                    cb = (uint32_t)((hi - lo) >> (32 * s));
                }
            } else if (lane == 0) {
                cb = (uint32_t)(chunk_bits_acc >> (32 * s));
            }
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
            const uint32_t twords = __shfl(incl, 63, 64);
            const uint64_t tbits = wave_sum_u64(cb);
            // ---- B (publish): this ticket's aggregate for stream s
            if (lane == 0) {
                __hip_atomic_store(&a.st[s].flags[T],
                                   make_flag(tag, T == 0 ? ST_PREFIX : ST_AGG, twords),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                S.twords[s] = twords;
                S.tbits[s] = tbits;
            }
        }
        __syncthreads();

        // ---- C: pack, stream by stream
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const StreamArgs& st = a.st[s];
            const uint32_t twords = S.twords[s];
            uint32_t TB = 0;      // S > 1: chunk-relative bit offset of the segment
            uint32_t carry = 0;   // S > 1: partial last word of the previous segment
            for (uint32_t g = 0; g < nseg; ++g) {
                const uint64_t i0 = tbeg + (uint64_t)g * SEG + (uint64_t)tid * SPT;
                const int nv = i0 >= tend ? 0 : (int)min<uint64_t>(SPT, tend - i0);
                uint64_t incl, own, seg_total = 0;
                if (nseg == 1) {
                    incl = S.incl[tid];
                    own = incl - (tid ? S.incl[tid - 1] : 0ull);
                } else {
                    // the segment's scan again (step A kept only totals)
                    load64<MODE>(a, i0, nv, w);
                    bool unused = false;
                    own = count_bits<NS>(S, w, nv, &unused);
                    incl = block_inclusive_scan(own, S.tmp, &seg_total);
                }
                const uint32_t mine = (uint32_t)(own >> (32 * s));  // this thread's bits
                uint32_t pos, ts, wc, ch;
                uint32_t r0 = 0, w0 = 0, touched;
                if (nseg == 1) {
                    ch = tid / L;
                    const uint64_t before = ch ? S.incl[ch * L - 1] : 0ull;
                    ts = (uint32_t)((incl - before) >> (32 * s)) - mine;  // chunk-relative start bit
                    wc = (S.cbits[s][min(ch, (uint32_t)MAX_G - 1)] + 31) >> 5;
                    pos = (ch < nch ? S.cword[s][ch] * 32u : 0u) + ts;
                    touched = twords;
                    for (uint32_t k = tid; k < touched; k += ENC_THREADS) S.stage[k] = 0u;
                } else {
                    ch = 0;
                    const uint32_t seg_bits = (uint32_t)(seg_total >> (32 * s));
                    const uint32_t excl = (uint32_t)(incl >> (32 * s)) - mine;
                    ts = TB + excl;
                    wc = (S.cbits[s][0] + 31) >> 5;
                    r0 = TB & 31u;
                    w0 = TB >> 5;
                    pos = r0 + excl;
                    touched = (r0 + seg_bits + 31) >> 5;
                    for (uint32_t k = tid; k <= touched; k += ENC_THREADS) S.stage[k] = k ? 0u : carry;
                    TB += seg_bits;
                }
                __syncthreads();
                if (nv == SPT && ch < nch)
                    pack64<true>(S, s, w[s], nv, pos, ts, wc, K, a.log2k, &S.gap[s][(ch * K) & (MAX_K - 1)]);
                else if (nv > 0 && ch < nch)
                    pack64<false>(S, s, w[s], nv, pos, ts, wc, K, a.log2k, &S.gap[s][(ch * K) & (MAX_K - 1)]);
                if (s == 0 && g == 0 && wave < NS) {
                    // ---- B (look-back), after the first packing: by now more of
                    // the tickets before this one have published prefixes
                    const int sl = wave;
                    const StreamArgs& sa = a.st[sl];
                    const uint32_t tw = S.twords[sl];
                    bool timed_out = false;
                    const uint64_t excl = T == 0 ? 0 : look_back(sa.flags, (int64_t)T, tag, &timed_out);
                    if (lane == 0) {
                        if (timed_out) set_status(sa.ws, LECB_ERR_WORKSPACE);
                        if (T) {
                            __hip_atomic_store(&sa.flags[T], make_flag(tag, ST_PREFIX, excl + tw),
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        }
                        S.tbase[sl] = excl;
                        atomicAdd(reinterpret_cast<unsigned long long*>(&sa.ws->bits),
                                  (unsigned long long)S.tbits[sl]);
                        if (T == a.ntickets - 1) {
                            __hip_atomic_store(&sa.ws->words, excl + tw, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                        }
                        if (S.uncoded) set_status(sa.ws, LECB_ERR_UNCODED_SYMBOL);
                        if (excl + tw >= (1ull << 32)) set_status(sa.ws, LECB_ERR_TOO_LARGE);
                        else if (excl + tw > sa.capacity_words) set_status(sa.ws, LECB_ERR_CAPACITY);
                    }
                    if (lane < (int)nch)
                        sa.table[c0 + lane] =
                            (uint32_t)(excl + S.cword[sl][lane] + ((S.cbits[sl][lane] + 31) >> 5));
                }
                __syncthreads();  // stage complete (and, the first time, the ticket bases known)
                const uint64_t tbase = S.tbase[s];
                const bool write_ok = tbase + twords <= st.capacity_words && !S.uncoded;
                if (nseg == 1) {
                    if (write_ok) {
                        uint32_t* dst = st.payload + tbase;
                        for (uint32_t k = tid; k < twords; k += ENC_THREADS) dst[k] = S.stage[k];
                    }
                } else {
                    const bool last_seg = g + 1 == nseg;
                    const uint32_t full = TB / 32 - w0;  // words completed by this segment
                    const uint32_t nwrite = last_seg ? touched : full;
                    if (write_ok) {
                        uint32_t* dst = st.payload + tbase + w0;
                        for (uint32_t k = tid; k < nwrite; k += ENC_THREADS) dst[k] = S.stage[k];
                    }
                    carry = S.stage[full];
                }
                __syncthreads();
            }
            // unit gaps of the ticket's chunks, K nibbles each
            if (K >= 2) {
                const uint32_t nbytes = nch * K / 2;
                for (uint32_t b = tid; b < nbytes; b += ENC_THREADS)
                    st.gaps[c0 * (K / 2) + b] = (uint8_t)(S.gap[s][2 * b] | (S.gap[s][2 * b + 1] << 4));
            } else {
                // one unit per chunk, gap 0; two chunks per byte (c0 is even)
                for (uint32_t b = tid; b < (nch + 1) / 2; b += ENC_THREADS) st.gaps[c0 / 2 + b] = 0;
            }
            if (c0 + nch == a.nc) {
                for (uint64_t b = st.table_pad_from + tid; b < st.table_pad_to; b += ENC_THREADS)
                    st.stream[b] = 0;
                for (uint64_t b = st.gap_pad_from + tid; b < st.gap_pad_to; b += ENC_THREADS)
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
            ws0->ticket = 0;
            const uint32_t ep = ws0->epoch;
            ws0->epoch = ep + 1;
            __threadfence();
            __hip_atomic_store(&ws0->exit_count, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

int launch_encode(const EncodeLaunch& L, void* stream) {
    EncArgs a{};
    a.in = L.in;
    a.n = L.n;
    a.chunk = L.chunk;
    a.log2k = (uint32_t)ilog2(units_per_chunk(L.chunk));
    a.nc = L.nc;
    a.G = L.chunk >= SEG ? 1u : SEG / L.chunk;
    a.S = L.chunk > SEG ? L.chunk / SEG : 1u;
    a.ntickets = (L.nc + a.G - 1) / a.G;
    const int ns = L.mode == ENC_PAIR ? 2 : 1;
    const uint64_t tb = table_bytes(L.nc), gb = gap_bytes(L.nc, L.chunk);
    for (int s = 0; s < ns; ++s) {
        StreamArgs& st = a.st[s];
        st.cb = L.st[s].cb;
        st.stream = L.st[s].out;
        st.table = reinterpret_cast<uint32_t*>(L.st[s].out);
        st.gaps = L.st[s].out + tb;
        st.payload = reinterpret_cast<uint32_t*>(L.st[s].out + tb + gb);
        st.header_bytes = tb + gb;
        st.capacity_words = (L.st[s].capacity - (tb + gb)) / 4;
        st.table_pad_from = 4 * L.nc;
        st.table_pad_to = tb;
        st.gap_pad_from = tb + (L.nc * units_per_chunk(L.chunk) + 1) / 2;
        st.gap_pad_to = tb + gb;
        st.res = L.st[s].res;
        st.ws = L.st[s].ws;
        st.flags = reinterpret_cast<uint64_t*>(L.st[s].ws + 1);
    }
    const uint64_t nwg = (uint64_t)L.grid < a.ntickets ? (uint64_t)L.grid : a.ntickets;
    const dim3 grid((uint32_t)nwg), block(ENC_THREADS);
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    switch (L.mode) {
        case ENC_BYTES: hipLaunchKernelGGL(encode_kernel<ENC_BYTES>, grid, block, 0, hs, a); break;
        case ENC_PLANE_LO: hipLaunchKernelGGL(encode_kernel<ENC_PLANE_LO>, grid, block, 0, hs, a); break;
        case ENC_PLANE_HI: hipLaunchKernelGGL(encode_kernel<ENC_PLANE_HI>, grid, block, 0, hs, a); break;
        case ENC_PAIR: hipLaunchKernelGGL(encode_kernel<ENC_PAIR>, grid, block, 0, hs, a); break;
        default: return LECB_ERR_INVALID_ARG;
    }
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

}  // namespace lecb
