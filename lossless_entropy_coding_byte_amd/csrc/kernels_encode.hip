// Huffman encode of byte symbols into stream format v1, in ONE launch.
//
// "Single-Stage Huffman Encoder for ML Compression", Methodology step 4: each
// tensor is coded directly with the codebook already resident on the device.
// "Lossless Compression for LLM Tensor Incremental Snapshots", Technical
// framework step 3 (Huffman coding of the byte groups) -- the plane variants
// read one byte plane straight out of the 16-bit words.
//
// One 256-thread workgroup owns one ticket at a time: a run of G consecutive
// chunks holding max(chunk, 16384) symbols (persistent grid; tickets come from
// an atomic counter, so every ticket a workgroup waits on is owned by a
// running workgroup).  Per ticket:
//   A. sum the code lengths per chunk -> payload words of each chunk (every
//      chunk starts on a word).  The input of up to GROUP_TILES tiles is
//      loaded with all loads in flight at once and stays in registers for
//      step C when the ticket fits in one such group;
//   B. decoupled look-back over the tickets before it -> first payload word
//      of the ticket.  Flags are 64-bit {epoch tag, state, value}, so no call
//      ever clears them; the look-back waits only on the tickets nearer than
//      the nearest published inclusive prefix;
//   C. per chunk, per tile of 4096 symbols: exclusive scan of per-thread bit
//      counts, every thread ORs its code words into an LDS staging buffer, the
//      finished words go out with coalesced stores, the partial last word is
//      carried to the next tile; the thread whose bit range holds a unit
//      boundary walks its code words to find that unit's gap.
#include <hip/hip_runtime.h>

#include "lecb_internal.hpp"

namespace lecb {

namespace {

constexpr int ENC_THREADS = 256;
constexpr int SYMS_PER_THREAD = 16;
constexpr int TILE = ENC_THREADS * SYMS_PER_THREAD;   // 4096 symbols
constexpr int STAGE_WORDS = TILE * 16 / 32 + 4;        // worst case 16 bits/symbol + carry
constexpr int GROUP_TILES = 4;                         // tiles held in registers at once
constexpr uint32_t TICKET_SYMBOLS = GROUP_TILES * TILE; // a ticket holds max(chunk, this)
constexpr int MAX_G = TICKET_SYMBOLS / 256;             // chunks per ticket at the smallest chunk
constexpr uint64_t FLAG_VALUE_MASK = (1ull << 34) - 1;
constexpr uint32_t ST_AGG = 1, ST_PREFIX = 2;

struct EncArgs {
    const uint8_t* in8;
    const uint16_t* in16;
    int plane;
    uint64_t n;
    uint32_t chunk;
    uint32_t log2k;
    uint64_t nc;
    uint32_t G;           // chunks per ticket
    uint64_t ntickets;
    const DeviceCodebook* cb;
    uint32_t* table;
    uint8_t* gaps;
    uint32_t* payload;
    uint64_t header_bytes;
    uint64_t payload_capacity_words;
    uint64_t table_pad_from, table_pad_to;  // byte range of table padding
    uint64_t gap_pad_from, gap_pad_to;      // byte range of gap padding (relative to stream)
    uint8_t* stream;
    lecb_result* res;
    WsHeader* ws;
    uint64_t* flags;
};

__device__ inline uint32_t lo_plane(uint32_t a, uint32_t b) {
    return (a & 0xFFu) | ((a >> 8) & 0xFF00u) | ((b & 0xFFu) << 16) | ((b << 8) & 0xFF000000u);
}
__device__ inline uint32_t hi_plane(uint32_t a, uint32_t b) {
    return ((a >> 8) & 0xFFu) | ((a >> 16) & 0xFF00u) | ((b << 8) & 0xFF0000u) | (b & 0xFF000000u);
}

// Symbol k of a thread's 16 (little-endian in w[4]).
__device__ inline uint32_t sym_of(const uint32_t w[4], int k) {
    return (w[k >> 2] >> (8 * (k & 3))) & 0xFFu;
}

// 16 symbols starting at i0 (valid below iend) packed little-endian into w[4];
// PLANE < 0: bytes, 0: low byte of 16-bit words, 1: high byte.
template <int PLANE>
__device__ inline void load16(const EncArgs& a, uint64_t i0, uint64_t iend, uint32_t w[4]) {
    if (i0 + 16 <= iend) {
        if constexpr (PLANE < 0) {
            const uint4 v = *reinterpret_cast<const uint4*>(a.in8 + i0);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else {
            const uint4 v0 = *reinterpret_cast<const uint4*>(a.in16 + i0);
            const uint4 v1 = *reinterpret_cast<const uint4*>(a.in16 + i0 + 8);
            if constexpr (PLANE == 1) {
                w[0] = hi_plane(v0.x, v0.y); w[1] = hi_plane(v0.z, v0.w);
                w[2] = hi_plane(v1.x, v1.y); w[3] = hi_plane(v1.z, v1.w);
            } else {
                w[0] = lo_plane(v0.x, v0.y); w[1] = lo_plane(v0.z, v0.w);
                w[2] = lo_plane(v1.x, v1.y); w[3] = lo_plane(v1.z, v1.w);
            }
        }
    } else {
        w[0] = w[1] = w[2] = w[3] = 0;
        for (int k = 0; k < 16; ++k) {
            if (i0 + k < iend) {
                uint32_t b;
                if constexpr (PLANE < 0) b = a.in8[i0 + k];
                else b = PLANE ? (a.in16[i0 + k] >> 8) : (a.in16[i0 + k] & 0xFF);
                w[k >> 2] |= b << (8 * (k & 3));
            }
        }
    }
}

// Input of GROUP_TILES consecutive tiles (thread's 16 symbols of each, tile t
// at i0 + t*TILE).  `full`: every one of them lies below iend; then all loads
// are issued before the first is used.
template <int PLANE>
__device__ inline void load_group(const EncArgs& a, uint64_t i0, uint64_t iend, bool full,
                                  uint32_t w[GROUP_TILES][4]) {
    if (full) {
        if constexpr (PLANE < 0) {
            uint4 v[GROUP_TILES];
#pragma unroll
            for (int t = 0; t < GROUP_TILES; ++t)
                v[t] = *reinterpret_cast<const uint4*>(a.in8 + i0 + (uint64_t)t * TILE);
#pragma unroll
            for (int t = 0; t < GROUP_TILES; ++t) {
                w[t][0] = v[t].x; w[t][1] = v[t].y; w[t][2] = v[t].z; w[t][3] = v[t].w;
            }
        } else {
            uint4 v0[GROUP_TILES], v1[GROUP_TILES];
#pragma unroll
            for (int t = 0; t < GROUP_TILES; ++t) {
                v0[t] = *reinterpret_cast<const uint4*>(a.in16 + i0 + (uint64_t)t * TILE);
                v1[t] = *reinterpret_cast<const uint4*>(a.in16 + i0 + (uint64_t)t * TILE + 8);
            }
#pragma unroll
            for (int t = 0; t < GROUP_TILES; ++t) {
                if constexpr (PLANE == 1) {
                    w[t][0] = hi_plane(v0[t].x, v0[t].y); w[t][1] = hi_plane(v0[t].z, v0[t].w);
                    w[t][2] = hi_plane(v1[t].x, v1[t].y); w[t][3] = hi_plane(v1[t].z, v1[t].w);
                } else {
                    w[t][0] = lo_plane(v0[t].x, v0[t].y); w[t][1] = lo_plane(v0[t].z, v0[t].w);
                    w[t][2] = lo_plane(v1[t].x, v1[t].y); w[t][3] = lo_plane(v1[t].z, v1[t].w);
                }
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < GROUP_TILES; ++t) load16<PLANE>(a, i0 + (uint64_t)t * TILE, iend, w[t]);
    }
}

__device__ inline uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ inline uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Exclusive scan of one value per thread over the 256-thread block.
// Returns the exclusive prefix; *total receives the block sum.
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_tmp[wave] = incl;
    __syncthreads();
    uint32_t before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < ENC_THREADS / 64; ++w) {
        const uint32_t x = s_tmp[w];
        if (w < wave) before += x;
        sum += x;
    }
    *total = sum;
    __syncthreads();  // s_tmp may be reused right after
    return before + incl - v;
}

__device__ inline uint64_t make_flag(uint32_t tag, uint32_t state, uint64_t value) {
    return ((uint64_t)tag << 36) | ((uint64_t)state << 34) | (value & FLAG_VALUE_MASK);
}

// Bound on polling rounds while waiting for a predecessor's flag.  Owners of
// earlier chunks publish within microseconds; only a workspace that was not
// zero-filled (stale ticket counter) could leave a flag unpublished, and then
// the call gives up with status WORKSPACE instead of waiting forever.
constexpr uint32_t SPIN_LIMIT = 1u << 24;

// Exclusive prefix (in payload words) of ticket c; run by all 64 lanes of
// wave 0.  Lane l watches ticket end-1-l.  A round is complete once every
// ticket nearer than the nearest inclusive prefix (state PREFIX) in the
// window is published; then their values, and that prefix, are added up.
// With no prefix in the window all 64 aggregates are added and the window
// moves down.  *timed_out is set when SPIN_LIMIT was reached.
__device__ uint64_t look_back(uint64_t* flags, int64_t c, uint32_t tag, bool* timed_out) {
    const int lane = threadIdx.x & 63;
    uint64_t excl = 0;
    int64_t end = c;
    uint32_t spins = 0;
    while (end > 0) {
        const int64_t idx = end - 1 - lane;
        uint64_t f = make_flag(tag, ST_PREFIX, 0);  // before ticket 0: prefix 0
        bool have = idx < 0;
        uint64_t pm, vm;
        for (;;) {
            if (!have) {
                f = __hip_atomic_load(&flags[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                have = (uint32_t)(f >> 36) == tag && ((f >> 34) & 3u) != 0;
            }
            pm = __ballot(have && ((f >> 34) & 3u) == ST_PREFIX);
            vm = __ballot(have);
            // lanes up to and including the nearest prefix must be published
            const uint64_t need = pm ? (pm ^ (pm - 1)) : ~0ull;
            if ((vm & need) == need) break;
            if (++spins >= SPIN_LIMIT) {
                *timed_out = true;
                return excl;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        const int stop = pm ? (int)__builtin_ctzll(pm) : 64;
        excl += wave_sum_u64(lane <= stop ? (f & FLAG_VALUE_MASK) : 0ull);
        if (pm) break;
        end -= 64;
    }
    return excl;
}

__device__ inline void set_status(WsHeader* ws, int32_t code) {
    atomicCAS(&ws->status, 0, code);
}

template <int PLANE>
__global__ __launch_bounds__(ENC_THREADS) void encode_kernel(EncArgs a) {
    __shared__ uint32_t s_enc[256];
    __shared__ uint32_t s_stage[STAGE_WORDS];
    __shared__ uint8_t s_gap[256];
    __shared__ uint32_t s_cbits[MAX_G];   // bits of each chunk of the ticket
    __shared__ uint32_t s_cword[MAX_G];   // first payload word of each chunk, ticket-relative
    __shared__ uint32_t s_tmp[8];
    __shared__ uint64_t s_bcast[3];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    s_enc[tid] = a.cb->enc[tid];
    if (tid == 0) {
        const uint32_t e = __hip_atomic_load(&a.ws->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_bcast[1] = (e % 0x0FFFFFFFu) + 1;
    }
    __syncthreads();
    const uint32_t tag = (uint32_t)s_bcast[1];
    const uint32_t K = 1u << a.log2k;
    const uint32_t G = a.G;

    for (;;) {
        if (tid == 0) s_bcast[0] = atomicAdd(&a.ws->ticket, 1u);
        if (tid < MAX_G) s_cbits[tid] = 0;
        __syncthreads();
        const uint64_t T = s_bcast[0];
        __syncthreads();
        if (T >= a.ntickets) break;

        const uint64_t c0 = T * G;                                  // first chunk
        const uint32_t nch = (uint32_t)min<uint64_t>(G, a.nc - c0);  // chunks in the ticket
        const uint64_t gbeg = c0 * a.chunk;
        const uint64_t gend = min(gbeg + (uint64_t)G * a.chunk, a.n);
        const uint32_t ntiles = (uint32_t)((gend - gbeg + TILE - 1) / TILE);
        const uint32_t ngroups = (ntiles + GROUP_TILES - 1) / GROUP_TILES;
        const uint64_t ti0 = gbeg + (uint64_t)tid * SYMS_PER_THREAD;  // this thread's symbols in tile 0

        // ---- A: bits of every chunk of the ticket
        uint32_t gw[GROUP_TILES][4];
        bool uncoded = false;
        for (uint32_t g = 0; g < ngroups; ++g) {
            const uint64_t rbeg = gbeg + (uint64_t)g * TICKET_SYMBOLS;
            const bool full = rbeg + TICKET_SYMBOLS <= gend;
            load_group<PLANE>(a, ti0 + (uint64_t)g * TICKET_SYMBOLS, gend, full, gw);
#pragma unroll
            for (int t = 0; t < GROUP_TILES; ++t) {
                const uint64_t i0 = ti0 + (uint64_t)(g * GROUP_TILES + t) * TILE;
                const int nvalid = full ? 16 : (i0 >= gend ? 0 : (int)min<uint64_t>(16, gend - i0));
                uint32_t bits = 0;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const uint32_t e = s_enc[sym_of(gw[t], k)];
                    if (k < nvalid) {
                        bits += e & 31u;
                        uncoded |= e == 0;
                    }
                }
                // a wave's 1024 symbols lie in one chunk when chunk >= 1024
                const uint32_t ci = (uint32_t)((i0 - gbeg) / a.chunk);
                if (a.chunk >= 1024) {
                    bits = wave_sum_u32(bits);
                    if (lane == 0 && bits) atomicAdd(&s_cbits[ci], bits);
                } else if (bits) {
                    atomicAdd(&s_cbits[ci], bits);
                }
            }
        }
        const int any_uncoded = __syncthreads_or(uncoded);
        // payload words of each chunk and their ticket-relative prefix (nch <= 64: wave 0)
        uint64_t twords = 0, tbits = 0;
        if (tid < 64) {
            const uint32_t cb = tid < (int)nch ? s_cbits[tid] : 0u;
            const uint32_t cw = (cb + 31) >> 5;
            uint32_t incl = cw;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t t = __shfl_up(incl, o, 64);
                if (lane >= o) incl += t;
            }
            if (tid < (int)nch) s_cword[tid] = incl - cw;
            twords = __shfl(incl, 63, 64);
            tbits = wave_sum_u64(cb);
            if (tid == 0) s_bcast[2] = twords;
        }

        // ---- B: decoupled look-back over tickets
        if (tid == 0) {
            __hip_atomic_store(&a.flags[T], make_flag(tag, T == 0 ? ST_PREFIX : ST_AGG, twords),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (tid < 64) {
            bool timed_out = false;
            const uint64_t excl = T == 0 ? 0 : look_back(a.flags, (int64_t)T, tag, &timed_out);
            if (tid == 0) {
                if (timed_out) set_status(a.ws, LECB_ERR_WORKSPACE);
                if (T) {
                    __hip_atomic_store(&a.flags[T], make_flag(tag, ST_PREFIX, excl + twords),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                s_bcast[0] = excl;
                atomicAdd(reinterpret_cast<unsigned long long*>(&a.ws->bits), (unsigned long long)tbits);
                if (T == a.ntickets - 1) {
                    __hip_atomic_store(&a.ws->words, excl + twords, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                if (any_uncoded) set_status(a.ws, LECB_ERR_UNCODED_SYMBOL);
                if (excl + twords >= (1ull << 32)) set_status(a.ws, LECB_ERR_TOO_LARGE);
                else if (excl + twords > a.payload_capacity_words) set_status(a.ws, LECB_ERR_CAPACITY);
            }
        }
        __syncthreads();
        const uint64_t tbase = s_bcast[0];
        twords = s_bcast[2];
        const bool write_ok = tbase + twords <= a.payload_capacity_words && !any_uncoded;
        if (tid < (int)nch) {
            const uint32_t cw = (s_cbits[tid] + 31) >> 5;
            a.table[c0 + tid] = (uint32_t)(tbase + s_cword[tid] + cw);
        }

        // ---- C: pack chunk by chunk, tile by tile
        uint32_t loaded = ngroups == 1 ? 0u : 0xFFFFFFFFu;  // register group in gw
        for (uint32_t ch = 0; ch < nch; ++ch) {
            const uint64_t c = c0 + ch;
            const uint64_t cbeg = c * a.chunk;
            const uint64_t cend = min(cbeg + a.chunk, a.n);
            const uint32_t cbits = s_cbits[ch];
            const uint64_t wc = (cbits + 31) >> 5;
            const uint64_t base = tbase + s_cword[ch];
            const uint32_t t_first = (uint32_t)((cbeg - gbeg) / TILE);
            const uint32_t t_end = (uint32_t)((cend - gbeg + TILE - 1) / TILE);
            uint32_t TB = 0;      // chunk-relative bit offset of the current tile
            uint32_t carry = 0;   // bits of the partial word left by the previous tile
            for (uint32_t t = t_first; t < t_end; ++t) {
                const uint32_t rg = t / GROUP_TILES;
                if (rg != loaded) {
                    const uint64_t rbeg = gbeg + (uint64_t)rg * TICKET_SYMBOLS;
                    load_group<PLANE>(a, ti0 + (uint64_t)rg * TICKET_SYMBOLS, gend,
                                      rbeg + TICKET_SYMBOLS <= gend, gw);
                    loaded = rg;
                }
                const uint64_t i0 = ti0 + (uint64_t)t * TILE;
                const int nvalid = (i0 < cbeg || i0 >= cend) ? 0 : (int)min<uint64_t>(16, cend - i0);
                uint32_t e[16];
                uint32_t bits = 0;
                const uint32_t tw = t % GROUP_TILES;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    uint32_t s0 = sym_of(gw[0], k);
#pragma unroll
                    for (int q = 1; q < GROUP_TILES; ++q)
                        if (tw == (uint32_t)q) s0 = sym_of(gw[q], k);
                    e[k] = k < nvalid ? s_enc[s0] : 0u;
                    bits += e[k] & 31u;
                }
                uint32_t tile_bits;
                const uint32_t off = block_exclusive_scan(bits, s_tmp, &tile_bits);
                const uint32_t r0 = TB & 31u, w0 = TB >> 5;
                const uint32_t touched = (r0 + tile_bits + 31) >> 5;
                for (uint32_t k = tid; k <= touched; k += ENC_THREADS) s_stage[k] = k ? 0u : carry;
                __syncthreads();

                // pack 16 code words at stage bit r0 + off: a 64-bit accumulator
                // whose top `used` bits belong to earlier code words of the word
                // being filled; after every second code word its top word is ORed
                // into the stage (again and again until the word is complete: OR
                // is idempotent) and, once complete, the accumulator moves on.
                uint32_t pos = r0 + off;
                uint32_t widx = pos >> 5;
                uint32_t used = pos & 31u;
                uint64_t acc = 0;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const uint32_t len = e[k] & 31u;
                    const uint32_t code = e[k] >> 5;
                    used += len;
                    acc |= (uint64_t)code << ((64 - used) & 63);  // ends at bit `used` from the top
                    if (k & 1) {
                        atomicOr(&s_stage[widx], (uint32_t)(acc >> 32));
                        const bool full_word = used >= 32;
                        acc = full_word ? acc << 32 : acc;
                        widx += full_word ? 1u : 0u;
                        used &= 31u;
                    }
                }
                if (used) atomicOr(&s_stage[widx], (uint32_t)(acc >> 32));

                // gaps of the unit boundaries B_j = 32*floor(j*wc/K) inside this
                // thread's bit range [ts, te) of the chunk: distance from B_j to
                // the first code word starting at or after it
                {
                    const uint32_t ts = TB + off, te = ts + bits;
                    if (te > ts) {
                        const uint32_t W = (ts + 31) >> 5;  // first word boundary >= ts
                        uint32_t j = (uint32_t)(((uint64_t)W * K + wc - 1) / wc);
                        for (; j < K; ++j) {
                            const uint32_t bj = (uint32_t)(((uint64_t)j * wc) >> a.log2k) << 5;
                            if (bj >= te) break;
                            uint32_t p = ts;
#pragma unroll
                            for (int k = 0; k < 16; ++k) {
                                if (p < bj) p += e[k] & 31u;
                            }
                            s_gap[j] = (uint8_t)(p - bj);
                        }
                    }
                }
                __syncthreads();  // stage complete

                const bool last_tile = t + 1 == t_end;
                const uint32_t full_words = (r0 + tile_bits) >> 5;
                const uint32_t nwrite = last_tile ? touched : full_words;
                if (write_ok) {
                    uint32_t* dst = a.payload + base + w0;
                    for (uint32_t k = tid; k < nwrite; k += ENC_THREADS) dst[k] = s_stage[k];
                }
                carry = s_stage[full_words];
                TB += tile_bits;
                __syncthreads();
            }

            // unit gaps of this chunk, K nibbles
            if (K >= 2) {
                for (uint32_t j = tid; j < K / 2; j += ENC_THREADS)
                    a.gaps[c * (K / 2) + j] = (uint8_t)(s_gap[2 * j] | (s_gap[2 * j + 1] << 4));
            } else if (tid == 0) {
                a.gaps[c / 2] = 0;  // K == 1: the only gap is 0; two chunks share the byte
            }
            __syncthreads();  // s_gap reused by the next chunk
        }
        if (c0 + nch == a.nc) {
            for (uint64_t b = a.table_pad_from + tid; b < a.table_pad_to; b += ENC_THREADS)
                a.stream[b] = 0;
            for (uint64_t b = a.gap_pad_from + tid; b < a.gap_pad_to; b += ENC_THREADS)
                a.stream[b] = 0;
        }
        __syncthreads();
    }

    // ---- exit: the last workgroup publishes the result and resets the workspace
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const uint32_t done = __hip_atomic_fetch_add(&a.ws->exit_count, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            const uint64_t words = __hip_atomic_load(&a.ws->words, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t bits = __hip_atomic_load(&a.ws->bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int32_t st = __hip_atomic_load(&a.ws->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            a.res->bytes = a.header_bytes + 4 * words;
            a.res->payload_bits = bits;
            a.res->status = st;
            a.res->reserved = 0;
            a.ws->ticket = 0;
            a.ws->words = 0;
            a.ws->bits = 0;
            a.ws->status = 0;
            const uint32_t ep = a.ws->epoch;
            a.ws->epoch = ep + 1;
            __threadfence();
            __hip_atomic_store(&a.ws->exit_count, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

int launch_encode(const EncodeLaunch& L, void* stream) {
    EncArgs a{};
    a.plane = L.plane;
    a.in8 = L.plane < 0 ? reinterpret_cast<const uint8_t*>(L.in) : nullptr;
    a.in16 = L.plane >= 0 ? reinterpret_cast<const uint16_t*>(L.in) : nullptr;
    a.n = L.n;
    a.chunk = L.chunk;
    a.log2k = (uint32_t)ilog2(units_per_chunk(L.chunk));
    a.nc = L.nc;
    a.G = L.chunk >= TICKET_SYMBOLS ? 1u : TICKET_SYMBOLS / L.chunk;
    a.ntickets = (L.nc + a.G - 1) / a.G;
    a.cb = L.cb;
    const uint64_t tb = table_bytes(L.nc), gb = gap_bytes(L.nc, L.chunk);
    a.stream = L.out;
    a.table = reinterpret_cast<uint32_t*>(L.out);
    a.gaps = L.out + tb;
    a.payload = reinterpret_cast<uint32_t*>(L.out + tb + gb);
    a.header_bytes = tb + gb;
    a.payload_capacity_words = (L.capacity - (tb + gb)) / 4;
    a.table_pad_from = 4 * L.nc;
    a.table_pad_to = tb;
    a.gap_pad_from = tb + (L.nc * units_per_chunk(L.chunk) + 1) / 2;
    a.gap_pad_to = tb + gb;
    a.res = L.res;
    a.ws = L.ws;
    a.flags = reinterpret_cast<uint64_t*>(L.ws + 1);
    const uint64_t nwg = (uint64_t)L.grid < a.ntickets ? (uint64_t)L.grid : a.ntickets;
    const dim3 grid((uint32_t)nwg), block(ENC_THREADS);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (L.plane < 0) hipLaunchKernelGGL(encode_kernel<-1>, grid, block, 0, st, a);
    else if (L.plane == 0) hipLaunchKernelGGL(encode_kernel<0>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(encode_kernel<1>, grid, block, 0, st, a);
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

}  // namespace lecb
