// Huffman decode of stream format v1 back to bytes.
//
// Reverse path of "Lossless Compression for LLM Tensor Incremental
// Snapshots", Technical framework (read, Huffman-decode); the independent
// parallel tasks of its Key design item 3 are the decode units: every chunk
// is split into K = chunk/256 units whose exact starting code-word boundary
// is its word-aligned start plus the stored 4-bit gap.
//
// One lane per unit, 256 units per workgroup; K divides 256, so a chunk's
// units never straddle workgroups.  Per lane:
//   1. count the code words between its start and the next unit's start
//      (the chunk's last unit takes the remainder of the chunk's symbols);
//   2. exclusive scan of the counts inside each chunk -> output offsets;
//   3. decode again, storing the symbols.
// A code word is looked up with the next LUT_BITS bits in an LDS table;
// longer ones use the canonical per-length limits.  Every structural rule of
// the format is checked; a violation sets status CORRUPT.
#include <hip/hip_runtime.h>

#include "lecb_internal.hpp"

namespace lecb {

namespace {

constexpr int DEC_THREADS = 256;

struct DecArgs {
    const uint32_t* table;
    const uint8_t* gaps;
    const uint32_t* payload;
    uint64_t payload_words;   // words present in the caller's buffer
    const DeviceCodebook* cb;
    uint32_t chunk;
    uint32_t log2k;
    uint64_t n;
    uint64_t nc;
    uint64_t header_bytes;
    uint64_t table_pad_from, table_pad_to;   // stream bytes that must be zero
    uint64_t gap_pad_from, gap_pad_to;
    const uint8_t* stream;
    uint8_t* out;
    lecb_result* res;
    WsHeader* ws;
};

struct Tables {
    uint16_t lut[LUT_SIZE];
    uint32_t limit[17];
    uint32_t first[17];
    uint32_t base[17];
    uint8_t sorted[256];
};

struct Reader {
    const uint32_t* p;
    uint64_t limit;   // words readable
    uint64_t wi;      // next word to load
    uint64_t buf;     // pending bits, MSB first
    int nb;           // valid bits in buf

    __device__ inline uint32_t ld(uint64_t i) const { return i < limit ? p[i] : 0u; }
    __device__ inline void start(uint64_t word, uint32_t bit) {
        buf = (((uint64_t)ld(word) << 32) | ld(word + 1)) << bit;
        nb = 64 - (int)bit;
        wi = word + 2;
    }
    __device__ inline void refill() {
        if (nb < 32) {
            buf |= (uint64_t)ld(wi++) << (32 - nb);
            nb += 32;
        }
    }
};

// One code word: returns its length (0 = no code word matches) and the symbol.
__device__ inline uint32_t decode_one(const Tables& T, Reader& r, uint32_t& sym) {
    r.refill();
    const uint32_t e = T.lut[r.buf >> (64 - LUT_BITS)];
    uint32_t len;
    if (e) {
        len = e >> 8;
        sym = e & 0xFFu;
    } else {
        const uint32_t v = (uint32_t)(r.buf >> 48);
        len = 0;
        for (uint32_t l = LUT_BITS + 1; l <= 16; ++l) {
            if (v < T.limit[l]) {
                len = l;
                break;
            }
        }
        if (!len) return 0;
        sym = T.sorted[T.base[len] + (v >> (16 - len)) - T.first[len]];
    }
    r.buf <<= len;
    r.nb -= (int)len;
    return len;
}

__device__ inline uint32_t gap_of(const uint8_t* gaps, uint64_t i) {
    const uint8_t b = gaps[i >> 1];
    return (i & 1) ? (b >> 4) : (b & 0xFu);
}

__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(DecArgs a) {
    __shared__ Tables T;
    __shared__ uint32_t s_cnt[DEC_THREADS];
    __shared__ uint64_t s_bits[DEC_THREADS / 64];

    const int tid = threadIdx.x;
    for (int i = tid; i < LUT_SIZE; i += DEC_THREADS) T.lut[i] = a.cb->lut[i];
    if (tid < 17) {
        T.limit[tid] = a.cb->limit[tid];
        T.first[tid] = a.cb->first[tid];
        T.base[tid] = a.cb->base[tid];
    }
    T.sorted[tid] = a.cb->sorted[tid];
    __syncthreads();

    const uint32_t K = 1u << a.log2k;
    const uint64_t u = (uint64_t)blockIdx.x * DEC_THREADS + tid;
    const uint64_t c = u >> a.log2k;
    const uint32_t j = (uint32_t)(u & (K - 1));
    const bool active = c < a.nc;
    bool bad = false;

    uint64_t sw = 0, wc = 0;
    uint32_t start_bit = 0, end_bit = 0, m_c = 0;
    const bool last = j == K - 1;
    if (active) {
        sw = c ? a.table[c - 1] : 0;
        const uint64_t ew = a.table[c];
        if (ew <= sw || ew > a.payload_words || ew - sw > a.chunk / 2) bad = true;
        wc = bad ? 0 : ew - sw;
        m_c = (uint32_t)min<uint64_t>(a.chunk, a.n - c * a.chunk);
        const uint32_t sj = (uint32_t)(((uint64_t)j * wc) >> a.log2k) << 5;
        const uint32_t gj = gap_of(a.gaps, u);
        if (j == 0 && gj != 0) bad = true;
        start_bit = sj + gj;
        if (!last) {
            const uint32_t sj1 = (uint32_t)(((uint64_t)(j + 1) * wc) >> a.log2k) << 5;
            end_bit = sj1 + gap_of(a.gaps, u + 1);
        }
    }

    // ---- 1. count
    uint32_t cnt = 0;
    if (active && !last && !bad) {
        Reader r{a.payload, a.payload_words, 0, 0, 0};
        r.start(sw + (start_bit >> 5), start_bit & 31);
        uint32_t pos = start_bit, last_start = 0xFFFFFFFFu;
        const uint32_t sj1 = end_bit - gap_of(a.gaps, u + 1);
        while (pos < end_bit) {
            uint32_t sym;
            const uint32_t len = decode_one(T, r, sym);
            if (!len) {
                bad = true;
                break;
            }
            last_start = pos;
            pos += len;
            ++cnt;
        }
        if (!bad) {
            if (pos != end_bit) bad = true;
            // the stored gap must name the FIRST boundary at or after sj1
            if (end_bit != sj1 && last_start != 0xFFFFFFFFu && last_start >= sj1) bad = true;
        }
    }

    // ---- 2. exclusive scan of counts within each chunk (segments of K lanes)
    s_cnt[tid] = cnt;
    __syncthreads();
    for (uint32_t o = 1; o < DEC_THREADS; o <<= 1) {
        const uint32_t v = tid >= (int)o ? s_cnt[tid - o] : 0u;
        __syncthreads();
        s_cnt[tid] += v;
        __syncthreads();
    }
    const int seg0 = tid - (int)j;  // lane of unit 0 of this chunk
    const uint32_t before_seg = seg0 > 0 ? s_cnt[seg0 - 1] : 0u;
    const uint32_t out_off = s_cnt[tid] - cnt - before_seg;
    if (active) {
        if (last) {
            if (out_off > m_c) bad = true;
            else cnt = m_c - out_off;
        } else if (out_off + cnt > m_c) {
            bad = true;  // never store outside this chunk's slot
        }
    }

    // ---- 3. decode and store
    uint64_t used_bits = 0;
    if (active && !bad) {
        Reader r{a.payload, a.payload_words, 0, 0, 0};
        r.start(sw + (start_bit >> 5), start_bit & 31);
        uint8_t* dst = a.out + c * a.chunk + out_off;
        uint32_t pos = start_bit;
        for (uint32_t k = 0; k < cnt; ++k) {
            uint32_t sym;
            const uint32_t len = decode_one(T, r, sym);
            if (!len) {
                bad = true;
                break;
            }
            pos += len;
            dst[k] = (uint8_t)sym;
        }
        if (!bad && last) {
            // data must end inside the chunk's last word, followed by zero padding
            const uint64_t endw = (uint64_t)wc << 5;
            if (pos > endw || pos + 32 <= endw) bad = true;
            else {
                const uint32_t rest = (uint32_t)(endw - pos);
                r.refill();
                if (rest && (r.buf >> (64 - rest)) != 0) bad = true;
            }
        }
        used_bits = pos - start_bit;
    }

    // padding bytes of the header are part of the format
    if (blockIdx.x == 0) {
        for (uint64_t b = a.table_pad_from + tid; b < a.table_pad_to; b += DEC_THREADS)
            bad |= a.stream[b] != 0;
        for (uint64_t b = a.gap_pad_from + tid; b < a.gap_pad_to; b += DEC_THREADS)
            bad |= a.stream[b] != 0;
        if (tid == 0 && ((a.nc << a.log2k) & 1))
            bad |= (a.stream[a.gap_pad_from - 1] >> 4) != 0;
    }

    // ---- status, accounting, exit
    const uint64_t wsum = [&] {
        uint64_t v = used_bits;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        return v;
    }();
    if ((tid & 63) == 0) s_bits[tid >> 6] = wsum;
    const int any_bad = __syncthreads_or(bad);
    if (tid == 0) {
        uint64_t tot = 0;
        for (int w = 0; w < DEC_THREADS / 64; ++w) tot += s_bits[w];
        if (tot) atomicAdd(reinterpret_cast<unsigned long long*>(&a.ws->bits), (unsigned long long)tot);
        if (any_bad) atomicCAS(&a.ws->status, 0, (int32_t)LECB_ERR_CORRUPT);
        __threadfence();
        const uint32_t done = __hip_atomic_fetch_add(&a.ws->exit_count, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            const uint64_t bits = __hip_atomic_load(&a.ws->bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int32_t st = __hip_atomic_load(&a.ws->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t W = a.table[a.nc - 1];
            a.res->bytes = a.header_bytes + 4 * W;
            a.res->payload_bits = bits;
            a.res->status = (st == 0 && W != a.payload_words) ? (int32_t)LECB_ERR_CORRUPT : st;
            a.res->reserved = 0;
            a.ws->bits = 0;
            a.ws->status = 0;
            __threadfence();
            __hip_atomic_store(&a.ws->exit_count, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

int launch_decode(const DecodeLaunch& L, void* stream) {
    DecArgs a{};
    const uint64_t tb = table_bytes(L.nc), gb = gap_bytes(L.nc, L.chunk);
    a.table = reinterpret_cast<const uint32_t*>(L.stream_base);
    a.gaps = L.stream_base + tb;
    a.payload = reinterpret_cast<const uint32_t*>(L.stream_base + tb + gb);
    a.payload_words = (L.stream_bytes - tb - gb) / 4;
    a.cb = L.cb;
    a.chunk = L.chunk;
    a.log2k = (uint32_t)ilog2(units_per_chunk(L.chunk));
    a.n = L.n;
    a.nc = L.nc;
    a.header_bytes = tb + gb;
    a.stream = L.stream_base;
    a.table_pad_from = 4 * L.nc;
    a.table_pad_to = tb;
    a.gap_pad_from = tb + (L.nc * units_per_chunk(L.chunk) + 1) / 2;
    a.gap_pad_to = tb + gb;
    a.out = L.out;
    a.res = L.res;
    a.ws = L.ws;
    const uint64_t units = L.nc * units_per_chunk(L.chunk);
    const uint64_t grid = (units + DEC_THREADS - 1) / DEC_THREADS;
    hipLaunchKernelGGL(decode_kernel, dim3((uint32_t)grid), dim3(DEC_THREADS), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

}  // namespace lecb
