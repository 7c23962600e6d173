// Huffman encode of byte symbols into stream format v1, in ONE launch.
//
// "Single-Stage Huffman Encoder for ML Compression", Methodology step 4: each
// tensor is coded directly with the codebook already resident on the device.
// "Lossless Compression for LLM Tensor Incremental Snapshots", Technical
// framework step 3 (Huffman coding of the byte groups) -- the plane variants
// read one byte plane straight out of the 16-bit words.
//
// One 256-thread workgroup owns one chunk at a time (persistent grid, chunk
// tickets from an atomic counter so every chunk a workgroup waits on is owned
// by a running workgroup).  Per chunk:
//   A. sum the code lengths of its symbols -> payload words Wc;
//   B. decoupled look-back over the chunks before it (one wavefront reads 64
//      predecessors' flags per step) -> first payload word of the chunk;
//      flags are 64-bit {epoch tag, state, value} so no call ever clears them;
//   C. per tile of 4096 symbols: exclusive scan of per-thread bit counts,
//      every thread ORs its code words into an LDS staging buffer, the
//      finished words go out with coalesced stores, the partial last word is
//      carried to the next tile; code words that cover a word boundary record
//      that boundary's gap, from which the chunk's unit gaps are picked.
#include <hip/hip_runtime.h>

#include "lecb_internal.hpp"

namespace lecb {

namespace {

constexpr int ENC_THREADS = 256;
constexpr int SYMS_PER_THREAD = 16;
constexpr int TILE = ENC_THREADS * SYMS_PER_THREAD;   // 4096 symbols
constexpr int STAGE_WORDS = TILE * 16 / 32 + 4;        // worst case 16 bits/symbol + carry
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

// 16 symbols starting at i0 (valid below iend) packed little-endian into w[4].
__device__ inline void load16(const EncArgs& a, uint64_t i0, uint64_t iend, uint32_t w[4]) {
    if (i0 + 16 <= iend) {
        if (a.plane < 0) {
            const uint4 v = *reinterpret_cast<const uint4*>(a.in8 + i0);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else {
            const uint4 v0 = *reinterpret_cast<const uint4*>(a.in16 + i0);
            const uint4 v1 = *reinterpret_cast<const uint4*>(a.in16 + i0 + 8);
            if (a.plane) {
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
                if (a.plane < 0) b = a.in8[i0 + k];
                else b = a.plane ? (a.in16[i0 + k] >> 8) : (a.in16[i0 + k] & 0xFF);
                w[k >> 2] |= b << (8 * (k & 3));
            }
        }
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

constexpr int LB_SLOTS = 4;  // flags each lane examines per round: 256 predecessors per round

// Exclusive prefix (in payload words) of chunk c; run by all 64 lanes of wave 0.
// Each round covers the 256 chunks below `end`: slot i of lane l holds chunk
// end-1-(64*i+l), so a smaller (64*i+l) is a nearer predecessor.  The round
// waits until every flag in it is published, then adds up everything from the
// nearest inclusive prefix (state PREFIX) upwards; with no prefix in the
// window it adds all 256 aggregates and moves down.  *timed_out is set when
// SPIN_LIMIT was reached.
__device__ uint64_t look_back(uint64_t* flags, int64_t c, uint32_t tag, bool* timed_out) {
    const int lane = threadIdx.x & 63;
    uint64_t excl = 0;
    int64_t end = c;
    uint32_t spins = 0;
    while (end > 0) {
        uint64_t f[LB_SLOTS];
        uint32_t pending = 0;  // bit i: slot i not yet valid
#pragma unroll
        for (int i = 0; i < LB_SLOTS; ++i) {
            const int64_t idx = end - 1 - (64 * i + lane);
            if (idx >= 0) {
                pending |= 1u << i;
            } else {
                f[i] = make_flag(tag, ST_PREFIX, 0);  // before chunk 0: prefix 0
            }
        }
        for (;;) {
#pragma unroll
            for (int i = 0; i < LB_SLOTS; ++i) {
                if (pending & (1u << i)) {
                    const int64_t idx = end - 1 - (64 * i + lane);
                    f[i] = __hip_atomic_load(&flags[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if ((uint32_t)(f[i] >> 36) == tag && ((f[i] >> 34) & 3u) != 0) pending &= ~(1u << i);
                }
            }
            if (__all(pending == 0)) break;
            if (++spins >= SPIN_LIMIT) {
                *timed_out = true;
                return excl;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        // nearest PREFIX: smallest offset 64*i + lane among slots in state PREFIX
        int stop = 64 * LB_SLOTS;  // offset of the nearest prefix, or none
#pragma unroll
        for (int i = 0; i < LB_SLOTS; ++i) {
            const uint64_t pm = __ballot(((f[i] >> 34) & 3u) == ST_PREFIX);
            if (pm && stop == 64 * LB_SLOTS) stop = 64 * i + (int)__builtin_ctzll(pm);
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

__global__ __launch_bounds__(ENC_THREADS) void encode_kernel(EncArgs a) {
    __shared__ uint32_t s_enc[256];
    __shared__ uint32_t s_stage[STAGE_WORDS];
    __shared__ uint8_t s_gapw[STAGE_WORDS];
    __shared__ uint8_t s_gap[256];
    __shared__ uint32_t s_tmp[8];
    __shared__ uint64_t s_bcast[2];

    const int tid = threadIdx.x;
    s_enc[tid] = a.cb->enc[tid];
    if (tid == 0) {
        const uint32_t e = __hip_atomic_load(&a.ws->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_bcast[1] = (e % 0x0FFFFFFFu) + 1;
    }
    __syncthreads();
    const uint32_t tag = (uint32_t)s_bcast[1];
    const uint32_t K = 1u << a.log2k;

    for (;;) {
        if (tid == 0) s_bcast[0] = atomicAdd(&a.ws->ticket, 1u);
        __syncthreads();
        const uint64_t c = s_bcast[0];
        __syncthreads();
        if (c >= a.nc) break;

        const uint64_t cbeg = c * a.chunk;
        const uint64_t cend = min(cbeg + a.chunk, a.n);
        const uint32_t ntiles = (uint32_t)((cend - cbeg + TILE - 1) / TILE);

        // ---- A: total bits of the chunk
        uint32_t my_bits = 0;
        bool uncoded = false;
        for (uint32_t t = 0; t < ntiles; ++t) {
            const uint64_t i0 = cbeg + (uint64_t)t * TILE + (uint64_t)tid * SYMS_PER_THREAD;
            uint32_t w[4];
            load16(a, i0, cend, w);
            const int nvalid = i0 >= cend ? 0 : (int)min<uint64_t>(16, cend - i0);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint32_t len = s_enc[(w[k >> 2] >> (8 * (k & 3))) & 0xFFu] & 31u;
                if (k < nvalid) {
                    my_bits += len;
                    uncoded |= len == 0;
                }
            }
        }
        uint32_t chunk_bits;
        (void)block_exclusive_scan(my_bits, s_tmp, &chunk_bits);
        const int any_uncoded = __syncthreads_or(uncoded);
        const uint64_t wc = (chunk_bits + 31) >> 5;

        // ---- B: decoupled look-back
        if (tid == 0) {
            __hip_atomic_store(&a.flags[c], make_flag(tag, c == 0 ? ST_PREFIX : ST_AGG, wc),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (tid < 64) {
            bool timed_out = false;
            const uint64_t excl = c == 0 ? 0 : look_back(a.flags, (int64_t)c, tag, &timed_out);
            if (tid == 0) {
                if (timed_out) set_status(a.ws, LECB_ERR_WORKSPACE);
                if (c) {
                    __hip_atomic_store(&a.flags[c], make_flag(tag, ST_PREFIX, excl + wc),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                s_bcast[0] = excl;
                a.table[c] = (uint32_t)(excl + wc);
                atomicAdd(reinterpret_cast<unsigned long long*>(&a.ws->bits),
                          (unsigned long long)chunk_bits);
                if (c == a.nc - 1) {
                    __hip_atomic_store(&a.ws->words, excl + wc, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                if (any_uncoded) set_status(a.ws, LECB_ERR_UNCODED_SYMBOL);
                if (excl + wc >= (1ull << 32)) set_status(a.ws, LECB_ERR_TOO_LARGE);
                else if (excl + wc > a.payload_capacity_words) set_status(a.ws, LECB_ERR_CAPACITY);
            }
        }
        __syncthreads();
        const uint64_t base = s_bcast[0];
        const bool write_ok = base + wc <= a.payload_capacity_words && !any_uncoded;

        // ---- C: pack tile by tile
        uint32_t TB = 0;      // chunk-relative bit offset of the current tile
        uint32_t carry = 0;   // bits of the partial word left by the previous tile
        for (uint32_t t = 0; t < ntiles; ++t) {
            const uint64_t i0 = cbeg + (uint64_t)t * TILE + (uint64_t)tid * SYMS_PER_THREAD;
            uint32_t w[4];
            load16(a, i0, cend, w);
            const int nvalid = i0 >= cend ? 0 : (int)min<uint64_t>(16, cend - i0);
            uint32_t e[16];
            uint32_t bits = 0;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                e[k] = k < nvalid ? s_enc[(w[k >> 2] >> (8 * (k & 3))) & 0xFFu] : 0u;
                bits += e[k] & 31u;
            }
            uint32_t tile_bits;
            const uint32_t off = block_exclusive_scan(bits, s_tmp, &tile_bits);
            const uint32_t r0 = TB & 31u, w0 = TB >> 5;
            const uint32_t touched = (r0 + tile_bits + 31) >> 5;
            for (uint32_t k = tid; k <= touched; k += ENC_THREADS) s_stage[k] = k ? 0u : carry;
            __syncthreads();

            // pack 16 code words at stage bit r0 + off
            uint32_t pos = r0 + off;
            uint32_t widx = pos >> 5;
            uint32_t used = pos & 31u;
            uint64_t acc = 0;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint32_t len = e[k] & 31u;
                if (len) {
                    const uint32_t code = e[k] >> 5;
                    // gap of a word boundary covered by this code word
                    if (used == 0) s_gapw[widx] = 0;
                    else if (used + len > 32) s_gapw[widx + 1] = (uint8_t)(used + len - 32);
                    acc |= (uint64_t)code << (64 - used - len);
                    used += len;
                    if (used >= 32) {
                        atomicOr(&s_stage[widx], (uint32_t)(acc >> 32));
                        acc <<= 32;
                        used -= 32;
                        ++widx;
                    }
                }
            }
            if (used) atomicOr(&s_stage[widx], (uint32_t)(acc >> 32));
            __syncthreads();

            const bool last_tile = t + 1 == ntiles;
            const uint32_t full = (r0 + tile_bits) >> 5;
            const uint32_t nwrite = last_tile ? touched : full;
            if (write_ok) {
                uint32_t* dst = a.payload + base + w0;
                for (uint32_t k = tid; k < nwrite; k += ENC_THREADS) dst[k] = s_stage[k];
            }
            for (uint32_t j = tid; j < K; j += ENC_THREADS) {
                const uint32_t wj = (uint32_t)(((uint64_t)j * wc) >> a.log2k);
                const uint32_t bj = wj << 5;
                if (bj >= TB && bj < TB + tile_bits) s_gap[j] = s_gapw[wj - w0];
            }
            carry = s_stage[full];
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
        if (c == a.nc - 1) {
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
    hipLaunchKernelGGL(encode_kernel, dim3(L.grid), dim3(ENC_THREADS), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

}  // namespace lecb
