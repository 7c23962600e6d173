// Huffman encode of byte symbols into stream format v3, in three launches
// (count, offsets, pack).
//
// "Single-Stage Huffman Encoder for ML Compression", Methodology step 4: each
// tensor is coded directly with the codebook already resident on the device.
// "Lossless Compression for LLM Tensor Incremental Snapshots", Technical
// framework step 3 (Huffman coding of the byte groups): the plane modes read
// one byte plane straight out of 16-bit words, and the pair modes code two
// planes of the same elements in one pass (two streams, two codebooks); Key
// design item 3 (independent parallel tasks): the lanes of the format.
//
// One hardware lane codes one lane of the format (lane geometry: lanes.hpp).
// A wave's task is 4 rows of 16 lanes, i.e. 4/P row groups of 16/G chunks.
// The pack launch's waves split the tasks into contiguous ranges; the count
// launch, with more waves, splits every range into K equal sub-ranges (they
// end where the ranges end):
//   1. count: every lane sums the code lengths of its symbols, stores its
//      word count nw = ceil(bits / 32) in the stream, and every wave stores
//      the words of its sub-range (per stream) in the workspace;
//   2. offsets: one workgroup turns the sub-ranges' words into their first
//      payload words (exclusive scan) and checks the total against the
//      capacity;
//   3. pack: every wave walks its range task by task.  A chunk's first word
//      is the range's first word (its first sub-range's) plus the words of
//      the range's earlier chunks; the chunk's end goes to the table.  Every lane then runs the
//      decoder's read order in lock step with its group: before each pair
//      of symbols, the lanes that completed a word in the previous pair get
//      the next read positions of the chunk (a count over the group's lanes),
//      and a lane writes each word it completes to the position reserved for
//      it two reads earlier (or by the reads of words 0 and 1).  Input blocks
//      of 16 symbols are read with one 16-byte load per lane: the lanes of a
//      row read neighbouring blocks.
#include <hip/hip_runtime.h>

#include <atomic>

#include <type_traits>

#include "lanes.hpp"

namespace lecb {

namespace {

constexpr int ENC_THREADS = 256;                 // four independent waves
constexpr int ENC_WAVES = ENC_THREADS / 64;
constexpr int OFF_THREADS = 1024;
constexpr uint32_t STAGE_LANE_WORDS = 32;   // pack: staging ring words per lane of a group
constexpr uint32_t FLUSH_PAIRS = 16;        // pack: pairs between flushes of the staging ring (two blocks)
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

struct StreamArgs {
    const DeviceCodebook* cb;
    uint32_t* table;
    uint16_t* nw;                            // word count of every lane
    uint32_t* payload;
    uint64_t header_bytes;
    uint64_t capacity_words;
    uint64_t table_pad_from, table_pad_to;  // byte ranges of header padding
    uint64_t nw_pad_from, nw_pad_to;
    uint8_t* stream;
    lecb_result* res;
    WsHeader* ws;
    uint64_t* range_words;                   // count: words of each range; offsets: first word of each
};

struct EncArgs {
    const void* in;
    const void* in2;     // ENC_PAIR_XOR: symbols are the planes of in[i] ^ in2[i]
    uint64_t n;
    uint32_t chunk;
    uint32_t lg;         // log2 of the lanes per chunk
    uint64_t nc;
    uint64_t ntasks;     // tasks of chunks_per_task chunks
    uint32_t cpt;        // chunks per task
    uint32_t nranges;    // waves of the pack launch: range r of the tasks each
    uint32_t nsub;       // waves of the count launch: range r is its sub-ranges rK .. rK + K - 1
    uint32_t sub_per_range;   // K
    StreamArgs st[2];
};

constexpr bool pair32_mode(int m) { return m == ENC_PAIR32_HI || m == ENC_PAIR32_LO; }
template <int MODE> struct Streams { static constexpr int value = two_stream_mode(MODE) ? 2 : 1; };

__device__ inline uint32_t lo_plane(uint32_t a, uint32_t b) {
    return (a & 0xFFu) | ((a >> 8) & 0xFF00u) | ((b & 0xFFu) << 16) | ((b << 8) & 0xFF000000u);
}
__device__ inline uint32_t hi_plane(uint32_t a, uint32_t b) {
    return ((a >> 8) & 0xFFu) | ((a >> 16) & 0xFF00u) | ((b << 8) & 0xFF0000u) | (b & 0xFF000000u);
}
// Byte `b` of four 32-bit elements as one word (element 0 in the low byte).
__device__ inline uint32_t byte_of4(const uint4& e, uint32_t b) {
    const uint32_t sel = b | ((b + 4u) << 8) | 0x0C0C0000u;   // bytes b of (lo, hi); 0x0C = zero
    const uint32_t t01 = __builtin_amdgcn_perm(e.y, e.x, sel);
    const uint32_t t23 = __builtin_amdgcn_perm(e.w, e.z, sel);
    return __builtin_amdgcn_perm(t23, t01, 0x05040100u);
}

// Byte of element i that plane `plane` (0 or 1 of the mode's streams) codes.
template <int MODE>
__device__ inline uint32_t symbol_at(const EncArgs& a, uint64_t i, uint32_t plane) {
    if constexpr (MODE == ENC_BYTES) {
        return static_cast<const uint8_t*>(a.in)[i];
    } else if constexpr (pair32_mode(MODE)) {
        const uint32_t e = static_cast<const uint32_t*>(a.in)[i];
        const uint32_t b = (MODE == ENC_PAIR32_HI ? 3u : 1u) - plane;
        return (e >> (8 * b)) & 0xFFu;
    } else {
        uint32_t x = static_cast<const uint16_t*>(a.in)[i];
        if constexpr (MODE == ENC_PAIR_XOR) x ^= static_cast<const uint16_t*>(a.in2)[i];
        const bool low = MODE == ENC_PLANE_LO || (two_stream_mode(MODE) && plane == 1);
        return low ? (x & 0xFFu) : (x >> 8);
    }
}

// The 16 symbols of the block starting at element e0 for `plane`, little-endian
// in w[0..3]; cnt < 16 symbols valid (the rest zero) only in the tensor's last block.
template <int MODE>
__device__ inline void block_symbols(const EncArgs& a, uint64_t e0, uint32_t cnt, uint32_t plane, uint32_t (&w)[4]) {
    if (cnt == BLOCK) {
        if constexpr (MODE == ENC_BYTES) {
            const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.in) + e0);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else if constexpr (pair32_mode(MODE)) {
            const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(a.in) + e0);
            const uint32_t b = (MODE == ENC_PAIR32_HI ? 3u : 1u) - plane;
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = byte_of4(p[q], b);
        } else {
            const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.in) + e0);
            uint4 v0 = p[0], v1 = p[1];
            if constexpr (MODE == ENC_PAIR_XOR) {
                const uint4* p2 = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.in2) + e0);
                const uint4 u0 = p2[0], u1 = p2[1];
                v0.x ^= u0.x; v0.y ^= u0.y; v0.z ^= u0.z; v0.w ^= u0.w;
                v1.x ^= u1.x; v1.y ^= u1.y; v1.z ^= u1.z; v1.w ^= u1.w;
            }
            const bool low = MODE == ENC_PLANE_LO || (two_stream_mode(MODE) && plane == 1);
            w[0] = low ? lo_plane(v0.x, v0.y) : hi_plane(v0.x, v0.y);
            w[1] = low ? lo_plane(v0.z, v0.w) : hi_plane(v0.z, v0.w);
            w[2] = low ? lo_plane(v1.x, v1.y) : hi_plane(v1.x, v1.y);
            w[3] = low ? lo_plane(v1.z, v1.w) : hi_plane(v1.z, v1.w);
        }
    } else {
        w[0] = w[1] = w[2] = w[3] = 0;
        for (uint32_t q = 0; q < cnt; ++q) {
            const uint32_t s = symbol_at<MODE>(a, e0 + q, plane);
            if (q < 4) w[0] |= s << (8 * q);
            else if (q < 8) w[1] |= s << (8 * (q - 4));
            else if (q < 12) w[2] |= s << (8 * (q - 8));
            else w[3] |= s << (8 * (q - 12));
        }
    }
}

__device__ inline uint32_t sym_of(const uint32_t (&w)[4], int k) { return (w[k >> 2] >> (8 * (k & 3))) & 0xFFu; }

__device__ inline uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ inline void set_status(WsHeader* ws, int32_t code) { atomicCAS(&ws->status, 0, code); }

// Tasks of range r when T tasks are split over R ranges.
__device__ inline uint64_t range_first(uint64_t r, uint64_t T, uint64_t R) { return r * T / R; }

// Where this lane works in a task: chunk, lane of the chunk, plane, symbols.
struct Place {
    uint64_t c;       // chunk
    uint32_t j;       // lane of the chunk
    uint32_t plane;   // stream
    uint32_t m;       // symbols of the lane
    bool valid;       // c < nc
};

template <int P>
__device__ inline Place place_of(const EncArgs& a, uint64_t task, uint32_t lane) {
    const uint32_t r = lane >> 4, i = lane & 15u;
    Place pl;
    pl.plane = r % P;
    pl.c = task * a.cpt + (r / P) * (16u >> a.lg) + (i >> a.lg);
    pl.j = i & ((1u << a.lg) - 1u);
    pl.valid = pl.c < a.nc;
    const uint32_t mc = pl.valid ? (uint32_t)min<uint64_t>(a.chunk, a.n - pl.c * a.chunk) : 0u;
    const uint32_t G = 1u << a.lg, full = mc / BLOCK, rest = mc % BLOCK;
    const uint32_t whole = full > pl.j ? (full - pl.j + G - 1) >> a.lg : 0u;
    pl.m = whole * BLOCK + ((full & (G - 1)) == pl.j && rest ? rest : 0u);
    return pl;
}

// First element of block t of the lane.
__device__ inline uint64_t block_elem(const EncArgs& a, const Place& pl, uint32_t t) {
    return pl.c * a.chunk + ((uint64_t)(t << a.lg) + pl.j) * BLOCK;
}

// Launch 1: word counts of every lane, words of every sub-range.
template <int MODE>
__global__ __launch_bounds__(ENC_THREADS) void count_kernel(EncArgs a) {
    constexpr int P = Streams<MODE>::value;
    __shared__ uint8_t len[2][256];
    const int tid = threadIdx.x;
    const uint32_t lane = tid & 63;
#pragma unroll
    for (int s = 0; s < P; ++s) len[s][tid] = (uint8_t)(a.st[s].cb->enc[tid] & 31u);
    __syncthreads();
    const uint64_t r = (uint64_t)blockIdx.x * ENC_WAVES + (tid >> 6);   // sub-range
    const uint64_t t0 = range_first(r, a.ntasks, a.nsub), t1 = range_first(r + 1, a.ntasks, a.nsub);
    uint64_t words[2] = {0, 0}, bits_all[2] = {0, 0};
    bool unc = false;
    for (uint64_t tk = t0; tk < t1; ++tk) {
        const Place pl = place_of<P>(a, tk, lane);
        const uint8_t* ln = len[P == 1 ? 0 : pl.plane];
        uint32_t bits = 0, mn = 16;
        const uint32_t nb = (pl.m + BLOCK - 1) / BLOCK;
        // Blocks whole in every lane of the wave (all but the tensor's last
        // chunk's) in a loop of whole-block loads only, so that the waits
        // count the loads: the symbols of blocks t + 1 and t + 2 are in
        // flight while block t is counted.  (With the short blocks' byte
        // loads in the same loop every block waited for all loads: the
        // count of 1 GiB of int8 took ~6 % longer.)
        // (modes with four 16-byte loads per block pick their bytes from all
        // four at once, so a load in flight would need 16 more registers per
        // block: those keep the loop over every block at the end)
        constexpr bool FAST = MODE == ENC_BYTES || MODE == ENC_PAIR || MODE == ENC_PLANE_LO || MODE == ENC_PLANE_HI;
        const uint32_t nfw = FAST ? wave_min_u32(pl.m) / BLOCK : 0u;
        if constexpr (MODE == ENC_PAIR || MODE == ENC_PLANE_LO || MODE == ENC_PLANE_HI) {
            // 16-bit elements: a block is two 16-byte loads, kept as loaded
            // (the plane's bytes are picked at use, so the wait comes there);
            // two buffers, the next block's loads in flight (bf16, 512 Mi
            // elements: encode 1.245 -> 1.20 ms against picking the bytes at
            // the load)
            if (nfw) {
                uint4 r0[2], r1[2];
                auto load_raw = [&](uint32_t t, uint4 (&r)[2]) {
                    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.in) +
                                                                    block_elem(a, pl, t));
                    r[0] = p[0];
                    r[1] = p[1];
                };
                load_raw(0, r0);
                const bool low = MODE == ENC_PLANE_LO || (MODE == ENC_PAIR && pl.plane == 1);
                const uint32_t sel = low ? 0x06040200u : 0x07050301u;
                auto step = [&](uint32_t t, const uint4 (&cur)[2], uint4 (&ahead)[2]) {
                    load_raw(t + 1 < nfw ? t + 1 : nfw - 1, ahead);
                        // the plane's bytes of two elements: bytes 0 and 2 (low
                    // plane) or 1 and 3 (high plane) of each word, by one permute
                    uint32_t w[4];
                    w[0] = __builtin_amdgcn_perm(cur[0].y, cur[0].x, sel);
                    w[1] = __builtin_amdgcn_perm(cur[0].w, cur[0].z, sel);
                    w[2] = __builtin_amdgcn_perm(cur[1].y, cur[1].x, sel);
                    w[3] = __builtin_amdgcn_perm(cur[1].w, cur[1].z, sel);
                    const bool on = t < nfw;
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        const uint32_t l = ln[sym_of(w, k)];
                        bits += on ? l : 0u;
                        mn = on ? min(mn, l) : mn;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                };
                for (uint32_t t = 0; t < nfw; t += 2) {
                    step(t, r0, r1);
                    step(t + 1, r1, r0);
                }
            }
        } else if (FAST && nfw) {
            // Four buffers, block x in buf[x % 4]: step t loads block t and
            // counts block t - 3, so three blocks' loads are in flight and the
            // waits count them exactly (`vmcnt(3)`).  Every load is issued in
            // the loop (past the whole blocks it reads the last one again,
            // still in the caches): loads before the loop, or a rotation of
            // the buffers by copies, made the compiler wait for all loads at
            // the loop head or at every copy.  (Encode of 1 GiB of int8, one
            // box: 1190 -> 1169 us against two blocks ahead with the first
            // loads before the loop.)
            uint32_t b0[4] = {0, 0, 0, 0}, b1[4] = {0, 0, 0, 0}, b2[4] = {0, 0, 0, 0}, b3[4] = {0, 0, 0, 0};
            auto step = [&](uint32_t t, uint32_t (&ld)[4], const uint32_t (&cur)[4]) {
                block_symbols<MODE>(a, block_elem(a, pl, t < nfw ? t : nfw - 1), BLOCK, pl.plane, ld);
                const bool on = t >= 3 && t - 3 < nfw;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const uint32_t l = ln[sym_of(cur, k)];
                    bits += on ? l : 0u;
                    mn = on ? min(mn, l) : mn;
                }
                __builtin_amdgcn_sched_barrier(0);   // one load per block, not all at once
            };
            for (uint32_t t = 0; t < nfw + 3; t += 4) {
                step(t, b0, b1);
                step(t + 1, b1, b2);
                step(t + 2, b2, b3);
                step(t + 3, b3, b0);
            }
        }
        if constexpr (FAST) {
            // the rest of the lane's blocks (the tensor's last chunk), one by one
            for (uint32_t t = nfw; t < nb; ++t) {
                const uint32_t cnt = min(BLOCK, pl.m - t * BLOCK);
                uint32_t wt[4];
                block_symbols<MODE>(a, block_elem(a, pl, t), cnt, pl.plane, wt);
                for (uint32_t k = 0; k < cnt; ++k) {
                    const uint32_t l = ln[sym_of(wt, (int)k)];
                    bits += l;
                    mn = min(mn, l);
                }
            }
        } else {
            // every block, the loads of blocks t + 1 and t + 2 issued ahead
            uint32_t w[4] = {0, 0, 0, 0}, wn[4] = {0, 0, 0, 0};
            if (nb) block_symbols<MODE>(a, block_elem(a, pl, 0), min(BLOCK, pl.m), pl.plane, w);
            if (nb > 1) block_symbols<MODE>(a, block_elem(a, pl, 1), min(BLOCK, pl.m - BLOCK), pl.plane, wn);
            for (uint32_t t = 0; t < nb; ++t) {
                const uint32_t cnt = min(BLOCK, pl.m - t * BLOCK);
                uint32_t wnn[4] = {0, 0, 0, 0};
                if (t + 2 < nb)
                    block_symbols<MODE>(a, block_elem(a, pl, t + 2), min(BLOCK, pl.m - (t + 2) * BLOCK), pl.plane,
                                        wnn);
                if (cnt == BLOCK) {
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        const uint32_t l = ln[sym_of(w, k)];
                        bits += l;
                        mn = min(mn, l);
                    }
                } else {
                    for (uint32_t k = 0; k < cnt; ++k) {
                        const uint32_t l = ln[sym_of(w, (int)k)];
                        bits += l;
                        mn = min(mn, l);
                    }
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    w[k] = wn[k];
                    wn[k] = wnn[k];
                }
            }
        }
        unc |= mn == 0;
        const uint32_t nw = (bits + 31) >> 5;
        if (pl.valid) a.st[pl.plane].nw[(pl.c << a.lg) + pl.j] = (uint16_t)nw;
        words[0] += pl.plane ? 0u : nw;
        words[1] += pl.plane ? nw : 0u;
        bits_all[0] += pl.plane ? 0u : bits;
        bits_all[1] += pl.plane ? bits : 0u;
    }
    // words and bits per stream
#pragma unroll
    for (int s = 0; s < P; ++s) {
        const uint64_t wsum = wave_sum_u64(words[s]);
        const uint64_t bsum = wave_sum_u64(bits_all[s]);
        if (lane == 0) {
            a.st[s].range_words[r] = wsum;
            if (bsum) atomicAdd(reinterpret_cast<unsigned long long*>(&a.st[s].ws->bits), (unsigned long long)bsum);
        }
    }
    const bool any_unc = __ballot(unc) != 0;
    if (any_unc && lane == 0) {
#pragma unroll
        for (int s = 0; s < P; ++s) set_status(a.st[s].ws, LECB_ERR_UNCODED_SYMBOL);
    }
}

// Launch 2: first payload word of every range (exclusive scan of the ranges'
// words, one stream after the other), total words, capacity checks.
__global__ __launch_bounds__(OFF_THREADS) void offsets_kernel(EncArgs a, int ns) {
    __shared__ uint64_t part[OFF_THREADS / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int s = 0; s < ns; ++s) {
        const StreamArgs& st = a.st[s];
        uint64_t run = 0;
        for (uint32_t b = 0; b < a.nsub; b += OFF_THREADS) {
            const uint32_t i = b + tid;
            const uint64_t v = i < a.nsub ? st.range_words[i] : 0ull;
            uint64_t incl = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint64_t t = __shfl_up(incl, o, 64);
                if (lane >= o) incl += t;
            }
            if (lane == 63) part[wave] = incl;
            __syncthreads();
            uint64_t before = 0, total = 0;
#pragma unroll
            for (int w = 0; w < OFF_THREADS / 64; ++w) {
                before += w < wave ? part[w] : 0ull;
                total += part[w];
            }
            if (i < a.nsub) st.range_words[i] = run + before + incl - v;
            run += total;
            __syncthreads();
        }
        if (tid == 0) {
            st.ws->words = run;
            if (run >= (1ull << 32)) set_status(st.ws, LECB_ERR_TOO_LARGE);
            else if (run > st.capacity_words) set_status(st.ws, LECB_ERR_CAPACITY);
        }
    }
}

// Launch 3: pack (see the top of the file).
template <int MODE, int LG>
__global__ __launch_bounds__(ENC_THREADS) void pack_kernel(EncArgs a) {
    constexpr int P = Streams<MODE>::value;
    constexpr uint32_t G = 1u << LG;
    constexpr uint32_t RE = STAGE_LANE_WORDS * G;   // staging words of a group
    __shared__ uint32_t enc[2][256];   // code | len << 16
    __shared__ __attribute__((aligned(16))) uint32_t stage[ENC_WAVES][4][STAGE_LANE_WORDS * 16];
    const int tid = threadIdx.x;
    const uint32_t lane = tid & 63;
#pragma unroll
    for (int s = 0; s < P; ++s) {
        const uint32_t e = a.st[s].cb->enc[tid];
        enc[s][tid] = (e >> 5) | ((e & 31u) << 16);
    }
    __syncthreads();
    const uint64_t r = (uint64_t)blockIdx.x * ENC_WAVES + (tid >> 6);
    const uint64_t t0 = range_first(r, a.ntasks, a.nranges), t1 = range_first(r + 1, a.ntasks, a.nranges);
    const uint32_t my_plane = (lane >> 4) % P;
    // this lane's stream, picked by conditional moves (no index into the arguments)
    const bool second = P == 2 && my_plane == 1;
    const uint16_t* const nwt = second ? a.st[1].nw : a.st[0].nw;
    uint32_t* const table = second ? a.st[1].table : a.st[0].table;
    uint32_t* const payload = second ? a.st[1].payload : a.st[0].payload;
    WsHeader* const my_ws = second ? a.st[1].ws : a.st[0].ws;
    // a stream with a status already (a byte without a code word, too many
    // words) gets no payload
    const bool skip = __hip_atomic_load(&my_ws->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    // first payload word of the range: that of its first sub-range
    uint64_t base = (second ? a.st[1].range_words : a.st[0].range_words)[r * a.sub_per_range];
    const uint32_t* e_tab = enc[second ? 1 : 0];

    for (uint64_t tk = t0; tk < t1; ++tk) {
        const Place pl = place_of<P>(a, tk, lane);
        const uint32_t N = pl.valid ? nwt[(pl.c << LG) + pl.j] : 0u;
        // the chunk's words, its first word, the task's words (per stream)
        const uint32_t wc = group_sum<LG>(N);
        const uint64_t mine = (pl.j == G - 1) ? (uint64_t)wc << (32 * my_plane) : 0ull;
        uint64_t incl = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint64_t t = __shfl_up(incl, o, 64);
            if (lane >= (uint32_t)o) incl += t;
        }
        const uint64_t at_last = __shfl(incl, (int)(lane | (G - 1)), 64);
        const uint64_t task_words = __shfl(incl, 63, 64);
        const uint32_t cend = (uint32_t)(at_last >> (32 * my_plane));     // task-relative end of the chunk
        const uint64_t cstart = base + cend - wc;
        base += (uint32_t)(task_words >> (32 * my_plane));
        if (pl.valid && pl.j == 0) table[pl.c] = (uint32_t)(cstart + wc);
        uint32_t* const out = payload + cstart;

        // Reads of words 0 and 1, then the pairs.  STAGED: a completed word goes
        // to the group's staging ring in LDS (slot = payload word index mod the
        // ring size, so 4-word groups of the payload are 16-byte groups of the
        // ring), and before every second block the words below the group's lowest
        // unwritten position, up to a 16-byte boundary of the payload, go out
        // with 16-byte stores (a lane writes 4 consecutive words, the group's
        // lanes neighbouring groups of 4); when the positions reserved by the
        // next pairs could reach a slot not yet stored, the task is coded again
        // with direct stores of each word (the words stored so far are the
        // same).
        const bool wr = !skip && pl.valid;
        const uint32_t nblk = (wave_max_u32(pl.m) + BLOCK - 1) / BLOCK;
        uint32_t* const ring = &stage[tid >> 6][lane >> 4][((lane & 15u) >> LG) * RE];
        const uint32_t rbase = (uint32_t)cstart;   // (mod RE: the ring slot of the chunk's word 0)
        const uint32_t lj = lane & (G - 1);
        auto code_task = [&](auto staged_c) -> bool {
            constexpr bool STAGED = decltype(staged_c)::value;
            // Positions are payload word indices of the chunk plus rbase (mod
            // 2^32), so that a position's low bits are its ring slot.
            uint32_t b0, n0, b1, n1;
            group_count<LG>(N >= 1, b0, n0);
            group_count<LG>(N >= 2, b1, n1);
            // posA: position of the word being filled; posB: of the one read
            // after it; cons: the group's next position to read
            uint32_t posA = rbase + b0, posB = rbase + n0 + b1, cons = rbase + n0 + n1;
            uint32_t done = 0;        // words completed
            const int32_t last_word = (int32_t)N - 1;
            uint64_t crossed = 0;     // lanes that completed a word in the previous pair
            // the lane's uncompleted bits: the low `fill` bits of acc
            uint64_t acc = 0;
            uint32_t fill = 0, flushed = 0;   // flushed: chunk-relative
            auto put = [&](uint32_t pos, uint32_t word) {
                if constexpr (STAGED) ring[pos & (RE - 1)] = word;
                else if (wr) out[pos - rbase] = word;
            };
            // STAGED: store the group's completed words (those below the lowest
            // position still to be written; `all`: every word) up to the last
            // 16-byte boundary of the payload below them (`all`: all of them);
            // false when the next FLUSH_PAIRS pairs could overrun the ring
            auto flush = [&](bool all) -> bool {
                const uint32_t f = group_min<LG>((all ? cons : (done < N ? posA : cons)) - rbase);
                // [flushed, a): words before the first 16-byte boundary; [a, b):
                // whole 16-byte groups; [b, f): the rest, stored only by `all`
                const uint32_t a = min(f, flushed + ((0u - (rbase + flushed)) & 3u));
                const uint32_t b = a + ((f - a) & ~3u);
                __builtin_amdgcn_wave_barrier();
                for (uint32_t x = flushed + lj; __ballot(x < a); x += G)
                    if (x < a && wr) out[x] = ring[(rbase + x) & (RE - 1)];
                for (uint32_t x = a + 4 * lj; __ballot(x < b); x += 4 * G)
                    if (x < b && wr)
                        *reinterpret_cast<v4u*>(out + x) = *reinterpret_cast<const v4u*>(&ring[(rbase + x) & (RE - 1)]);
                if (all)
                    for (uint32_t x = b + lj; __ballot(x < f); x += G)
                        if (x < f && wr) out[x] = ring[(rbase + x) & (RE - 1)];
                flushed = all ? f : b;
                __builtin_amdgcn_wave_barrier();
                // the next pairs read at most one word per lane each, so their
                // puts stay below cons + FLUSH_PAIRS * G
                return __ballot(cons - rbase + FLUSH_PAIRS * G - flushed > RE) == 0;
            };
            // One block: its code words (the wait for its symbols), the flush of
            // the words completed so far (STAGED, `fl`: every second block;
            // every block measured 0.9 % (int8) to 2.4 % (bf16) slower, every
            // fourth overran the ring and fell back to direct stores), `ahead`
            // (the next block's load), the 8 pairs.  Global stores and loads
            // complete in order,
            // so a load's wait also waits for the stores issued before it: the
            // stores and the load both go out a whole block before the next
            // wait (measured 0.8 % faster on 1 GiB than the load after pair 3).
            // False when the staging would overrun.  (One body for whole and
            // short blocks: a second, whole-block copy needs about 20 more
            // VGPRs.)
            auto code_block = [&](const uint32_t (&w)[4], uint32_t cnt, auto&& ahead, bool fl) -> bool {
                uint32_t e[16];
#pragma unroll
                for (int k = 0; k < 16; ++k) e[k] = e_tab[sym_of(w, k)];
                // past the lane's symbols: no bits (only a lane's last block
                // is short, so the wave mostly skips this)
                if (__builtin_amdgcn_ballot_w64(cnt < BLOCK) != 0) {
#pragma unroll
                    for (int k = 0; k < 16; ++k) e[k] = (uint32_t)k < cnt ? e[k] : 0u;
                }
                if constexpr (STAGED) {
                    if (fl && !flush(false)) return false;
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    if (q == 0) ahead();
                    // before the pair: the lanes that completed a word read the
                    // next one (after a lane's last word no word is left to
                    // read), at the group's next positions in lane order (the
                    // loop runs with every lane active, so ballots see the wave)
                    const uint64_t fm = crossed & __builtin_amdgcn_ballot_w64((int32_t)done < last_word);
                    uint32_t below, total;
                    group_count_mask<LG>(fm, below, total);
                    posB = __builtin_amdgcn_inverse_ballot_w64(fm) ? cons + below : posB;
                    cons += total;
                    // the pair's code words (at most 32 bits) into the accumulator
                    const uint32_t e0 = e[2 * q], e1 = e[2 * q + 1];
                    const uint32_t l = (e0 >> 16) + (e1 >> 16);
                    const uint32_t c2 = ((e0 & 0xFFFFu) << (e1 >> 16)) | (e1 & 0xFFFFu);
                    acc = (acc << l) | c2;
                    fill += l;   // at most 31 + 32
                    const bool cr = fill >= 32;
                    crossed = __builtin_amdgcn_ballot_w64(cr);
                    fill &= 31u;
                    if (cr) {
                        put(posA, __builtin_amdgcn_alignbit((uint32_t)(acc >> 32), (uint32_t)acc, fill));
                        posA = posB;
                    }
                    done = plus_lane_bit(done, crossed);
                }
                return true;
            };
            // the lane's block t (symbols loaded during the block before)
            auto load = [&](uint32_t t, uint32_t (&w)[4]) -> uint32_t {
                const uint32_t cnt = pl.m > t * BLOCK ? min(BLOCK, pl.m - t * BLOCK) : 0u;
                w[0] = w[1] = w[2] = w[3] = 0;
                if (cnt) block_symbols<MODE>(a, block_elem(a, pl, t), cnt, pl.plane, w);
                return cnt;
            };
            uint32_t w[4], cnt = nblk ? load(0, w) : 0u;
            for (uint32_t t = 0; t < nblk; ++t) {
                uint32_t wn[4] = {0, 0, 0, 0}, cn = 0;
                if (!code_block(w, cnt, [&] {
                        if (t + 1 < nblk) cn = load(t + 1, wn);
                    }, (t & 1) == 0))
                    return true;
#pragma unroll
                for (int k = 0; k < 4; ++k) w[k] = wn[k];
                cnt = cn;
            }
            if (fill) put(posA, (uint32_t)(acc << (32 - fill)));
            if constexpr (STAGED) flush(true);
            return false;
        };
        if (code_task(std::true_type{})) code_task(std::false_type{});
        // header padding: the wave of the last task
        if (tk + 1 == a.ntasks) {
#pragma unroll
            for (int s = 0; s < P; ++s) {
                const StreamArgs& sa = a.st[s];
                for (uint64_t b = sa.table_pad_from + lane; b < sa.table_pad_to; b += 64) sa.stream[b] = 0;
                for (uint64_t b = sa.nw_pad_from + lane; b < sa.nw_pad_to; b += 64) sa.stream[b] = 0;
            }
        }
    }

    // ---- exit: the last wave publishes the results and resets the workspace
    if (lane == 0) {
        __threadfence();
        WsHeader* ws0 = a.st[0].ws;
        const uint32_t done = __hip_atomic_fetch_add(&ws0->exit_count, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == a.nranges - 1) {
#pragma unroll
            for (int s = 0; s < P; ++s) {
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

// Workgroups of an encode kernel resident on one CU (asked once per device,
// kernel (0 count, 1 pack), mode and lane count; concurrent first calls store
// the same value).
uint64_t workgroups_per_cu(int which, int mode, int lg, const void* kernel) {
    static std::atomic<int> cached[MAX_DEVICES][2][ENC_NUM_MODES][5];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return 4;
    int nb = cached[dev][which][mode][lg].load(std::memory_order_relaxed);
    if (!nb) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, ENC_THREADS, 0) != hipSuccess || nb <= 0)
            nb = 4;
        cached[dev][which][mode][lg].store(nb, std::memory_order_relaxed);
    }
    return (uint64_t)nb;
}

template <typename F>
hipError_t with_lg(uint32_t lg, F&& f) {
    switch (lg) {
        case 0: return f(std::integral_constant<int, 0>{});
        case 1: return f(std::integral_constant<int, 1>{});
        case 2: return f(std::integral_constant<int, 2>{});
        case 3: return f(std::integral_constant<int, 3>{});
        case 4: return f(std::integral_constant<int, 4>{});
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int launch_encode(const EncodeLaunch& L, void* stream) {
    if (L.mode < 0 || L.mode >= ENC_NUM_MODES) return LECB_ERR_INVALID_ARG;
    EncArgs a{};
    a.in = L.in;
    a.in2 = L.in2;
    a.n = L.n;
    a.chunk = L.chunk;
    a.lg = (uint32_t)ilog2(lanes_per_chunk(L.chunk));
    a.nc = L.nc;
    const int ns = two_stream_mode(L.mode) ? 2 : 1;
    a.cpt = (4u / (uint32_t)ns) * (16u >> a.lg);
    a.ntasks = (L.nc + a.cpt - 1) / a.cpt;
    for (int s = 0; s < ns; ++s)
        if (!L.st[s].cb || !L.st[s].out || !L.st[s].res || !L.st[s].ws) return LECB_ERR_INVALID_ARG;
    const uint64_t tb = table_bytes(L.nc), cb = count_bytes(L.nc, L.chunk);
    for (int s = 0; s < ns; ++s) {
        StreamArgs& st = a.st[s];
        st.cb = L.st[s].cb;
        st.stream = L.st[s].out;
        st.table = reinterpret_cast<uint32_t*>(L.st[s].out);
        st.nw = reinterpret_cast<uint16_t*>(L.st[s].out + tb);
        st.payload = reinterpret_cast<uint32_t*>(L.st[s].out + tb + cb);
        st.header_bytes = tb + cb;
        st.capacity_words = (L.st[s].capacity - (tb + cb)) / 4;
        st.table_pad_from = 4 * L.nc;
        st.table_pad_to = tb;
        st.nw_pad_from = tb + 2 * L.nc * lanes_per_chunk(L.chunk);
        st.nw_pad_to = tb + cb;
        st.res = L.st[s].res;
        st.ws = L.st[s].ws;
        st.range_words = reinterpret_cast<uint64_t*>(L.st[s].ws + 1);  // room for nc + 4 >= nsub values
    }
    // Ranges: one per wave of the pack launch, as many waves as the GPU holds
    // at once (workgroups of the pack kernel resident per CU, from its
    // registers and LDS) when there are tasks enough, never more ranges than
    // tasks beyond the last workgroup's padding.  Every wave then works from
    // the start to the end of the launch; a grid of more waves than fit ran a
    // second round that slowed the first one's last tasks (1 GiB of int8:
    // 1.64 -> 1.27 ms).  The count launch, which mostly waits for its loads,
    // splits every range into K sub-ranges (K equal parts of a range end
    // where the ranges end) for as many waves as the GPU holds of it, never
    // more sub-ranges than tasks; so at most nc + 3 values go to the
    // workspace, which holds nc + 4.
    const uint64_t cus = (uint64_t)device_cu_count();
    if (cus == 0) return LECB_ERR_HIP;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = with_mode(L.mode, [&](auto m) {
        constexpr int M = decltype(m)::value;
        return with_lg(a.lg, [&](auto g) {
            constexpr int LG = decltype(g)::value;
            const uint64_t per_cu = workgroups_per_cu(1, M, LG, reinterpret_cast<const void*>(&pack_kernel<M, LG>));
            const uint64_t count_per_cu = workgroups_per_cu(0, M, 0, reinterpret_cast<const void*>(&count_kernel<M>));
            uint64_t waves = cus * per_cu * ENC_WAVES;
            if (waves > a.ntasks) waves = a.ntasks;
            const uint64_t nwg = (waves + ENC_WAVES - 1) / ENC_WAVES;
            a.nranges = (uint32_t)(nwg * ENC_WAVES);
            uint64_t k = (cus * count_per_cu * ENC_WAVES + a.nranges - 1) / a.nranges;
            const uint64_t kmax = a.ntasks / a.nranges;
            if (k > kmax) k = kmax;
            if (k < 1) k = 1;
            a.sub_per_range = (uint32_t)k;
            a.nsub = (uint32_t)(a.nranges * k);
            const dim3 grid((uint32_t)nwg), block(ENC_THREADS);
            hipLaunchKernelGGL(count_kernel<M>, dim3((uint32_t)(nwg * k)), block, 0, hs, a);
            hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(OFF_THREADS), 0, hs, a, ns);
            hipLaunchKernelGGL((pack_kernel<M, LG>), grid, block, 0, hs, a);
            return hipSuccess;
        });
    });
    if (e != hipSuccess) return LECB_ERR_INVALID_ARG;
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

}  // namespace lecb
