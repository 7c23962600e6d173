// Huffman decode of stream format v1 back to bytes.
//
// Reverse path of "Lossless Compression for LLM Tensor Incremental
// Snapshots", Technical framework (read, Huffman-decode); the independent
// parallel tasks of its Key design item 3 are the decode units: every chunk
// is split into K = chunk/256 units whose exact starting code-word boundary
// is its word-aligned start plus the stored 4-bit gap.
//
// One lane per unit, 256 units per workgroup (K divides 256, so a chunk's
// units never straddle workgroups).  Per lane:
//   1. count pass: code words that start in [start, end) of the unit; the
//      loop stops exactly at `end`, which checks that `end` is a code-word
//      boundary and that the stored gap names the first one.  The chunk's
//      last unit counts only the code words that start before the chunk's
//      last payload word;
//   2. exclusive scan of the counts inside each chunk -> output offsets; the
//      last unit now knows how many code words remain in the last word,
//      decodes them and checks the zero padding behind them;
//   3. decode pass: output is written in whole DEC_BLOCK-byte blocks, aligned
//      within the chunk's output.  A lane owns the blocks that START inside
//      its output range; it skips the code words in front of its first block
//      (the previous lane's last block holds them) and decodes on past its
//      own end, into the next unit's code words, to fill its last block.
//      Blocks never cross a chunk (a chunk holds a multiple of 256 symbols),
//      and with a 32-byte aligned output buffer every store fills whole
//      32-byte sectors.
//
// Bit reader: a window of two payload words and a bit offset into it; before
// every pair of code words the window slides by one word when its first word
// is used up (no branch).  Afterwards the offset is below 32, so the window
// holds >= 33 bits, enough for two code words of at most 16 bits.  The words
// come from a per-lane ring of 16 payload words in LDS; the ring is topped up on a fixed
// schedule (every 4 refills) by one masked 32-byte global load whose data go
// into the ring at the next top-up, so the decode loop never waits on global
// memory.  Ring slot q of lane L sits at ring[q][L]: each lane has its own bank.
//
// A code word of at most LUT_BITS bits is one LDS lookup; longer ones use the
// canonical per-length limits.  Every structural rule of the format is
// checked; a violation sets status CORRUPT.
#include <hip/hip_runtime.h>

#include "lecb_internal.hpp"

namespace lecb {

namespace {

constexpr int DEC_MAX_THREADS = 1024;  // lanes (decode units) per workgroup: 256, 512 or 1024
constexpr uint32_t RING = 16;  // payload words per lane in LDS
constexpr uint32_t DEC_BLOCK = 32;  // output block a lane owns (bytes)
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

struct DecStream {
    const uint32_t* table;
    const uint8_t* gaps;
    const uint32_t* payload;
    uint64_t payload_words;   // words present in the caller's buffer
    const DeviceCodebook* cb;
    uint64_t header_bytes;
    uint64_t table_pad_from, table_pad_to;   // stream bytes that must be zero
    uint64_t gap_pad_from, gap_pad_to;
    const uint8_t* stream;
    uint8_t* out;
    lecb_result* res;
    WsHeader* ws;
};

struct DecArgs {
    const lecb_result* sizes;  // non-null: stream k's size is sizes[k].bytes (an encoder's result)
    uint32_t chunk;
    uint32_t log2k;
    uint64_t n;
    uint64_t nc;
    uint32_t wg_per_stream;   // workgroups of one stream; stream = blockIdx.x / wg_per_stream
    uint32_t nstreams;
    DecStream st[2];
};

struct Tables {
    uint16_t lut[LUT_SIZE];   // (sym << 8) | len
    uint8_t mlut[LUT_SIZE];   // (count << 4) | bits of the whole code words in the next LUT_BITS
    uint32_t off[17];         // base[l] - first[l]: index in `sorted` is off[l] + code
    uint8_t sorted[256];
};

// The tables come first: their LDS offsets (and the ring's base) fit the
// 16-bit offset field of the LDS instructions, so a table lookup needs no
// base-address add.
template <int NT>
struct Shared {
    Tables T;
    alignas(16) uint32_t ring[RING][NT];  // row 0 doubles as the counts of the scan
    uint64_t red[NT / 64];
};

// Left-aligned canonical limits of the lengths above LUT_BITS (uniform values).
struct Limits {
    uint32_t l13, l14, l15, l16;
};

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

// Next code word as (sym << 8) | len, len in 1..16, from the next 32 bits
// `top`.  An invalid code word yields len 16 and sets `inval`.
__device__ inline uint32_t lookup(const Tables& T, const Limits& L, uint32_t top, uint32_t& inval) {
    uint32_t e = T.lut[top >> (32 - LUT_BITS)];
    if (e == 0) {
        const uint32_t v = top >> 16;
        const uint32_t len = 13u + (v >= L.l13) + (v >= L.l14) + (v >= L.l15);
        if (v >= L.l16) {
            inval = 1;
            e = 16;
        } else {
            e = ((uint32_t)T.sorted[(T.off[len] + (v >> (16 - len))) & 255u] << 8) | len;
        }
    }
    return e;
}

// Decode one code word and advance; returns (sym << 8) | len.
template <int NT>
__device__ inline uint32_t step(const Tables& T, const Limits& L, Reader<NT>& r, uint32_t& inval) {
    const uint32_t e = lookup(T, L, r.peek(), inval);
    r.off += e & 0xFFu;
    return e;
}

// The symbols (byte 1) of four table entries as one little-endian word:
// two byte permutes gather the pairs, a third joins them.
__device__ inline uint32_t syms4(const uint32_t (&e)[4]) {
    const uint32_t p01 = __builtin_amdgcn_perm(e[1], e[0], 0x0c0c0501u);
    const uint32_t p23 = __builtin_amdgcn_perm(e[3], e[2], 0x0c0c0501u);
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}

__device__ inline uint32_t gap_of(const uint8_t* gaps, uint64_t i) {
    const uint8_t b = gaps[i >> 1];
    return (i & 1) ? (b >> 4) : (b & 0xFu);
}

// 64 VGPRs at most: two 1024-lane workgroups (8 waves per SIMD) fit a CU.
template <int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8, 8))) void decode_kernel(DecArgs a) {
    constexpr int DEC_THREADS = NT;
    __shared__ __attribute__((aligned(16))) Shared<NT> S;
    Tables& T = S.T;

    const int tid = threadIdx.x;
    const uint32_t sidx = blockIdx.x / a.wg_per_stream;
    const uint32_t bid = blockIdx.x - sidx * a.wg_per_stream;
    const DecStream& d0 = a.st[sidx];
    DecStream d = d0;
    bool size_bad = false;
    if (a.sizes) {
        // the stream's size comes from the encoder's result on the device
        const uint64_t bytes = a.sizes[sidx].bytes;
        size_bad = a.sizes[sidx].status != 0 || bytes < d.header_bytes + 4 ||
                   ((bytes - d.header_bytes) & 3) != 0;
        d.payload_words = size_bad ? 0 : (bytes - d.header_bytes) / 4;
    }
    {
        const v4u* src = reinterpret_cast<const v4u*>(d.cb->lut);
        v4u* dst = reinterpret_cast<v4u*>(T.lut);
        constexpr int NV = LUT_SIZE * 2 / 16;
        for (int i = tid; i < NV; i += DEC_THREADS) dst[i] = src[i];
        const v4u* msrc = reinterpret_cast<const v4u*>(d.cb->mlut);
        v4u* mdst = reinterpret_cast<v4u*>(T.mlut);
        for (int i = tid; i < LUT_SIZE / 16; i += DEC_THREADS) mdst[i] = msrc[i];
    }
    if (tid < 17) T.off[tid] = d.cb->base[tid] - d.cb->first[tid];
    if (tid < 256) T.sorted[tid] = d.cb->sorted[tid];
    Limits L;
    L.l13 = d.cb->limit[13];
    L.l14 = d.cb->limit[14];
    L.l15 = d.cb->limit[15];
    L.l16 = d.cb->limit[16];

    // ---- unit geometry
    const uint32_t K = 1u << a.log2k;
    const uint64_t u = (uint64_t)bid * DEC_THREADS + tid;
    const uint64_t c = u >> a.log2k;
    const uint32_t j = (uint32_t)(u & (K - 1));
    const bool active = c < a.nc && !size_bad;
    const bool last = j == K - 1;
    bool bad = size_bad;
    uint64_t sw = 0, wc = 0;
    uint32_t start_bit = 0, end_bit = 0, sj1 = 0, m_c = 0;
    if (active) {
        sw = c ? d.table[c - 1] : 0;
        const uint64_t ew = d.table[c];
        if (ew <= sw || ew > d.payload_words || ew - sw > a.chunk / 2) bad = true;
        wc = bad ? 0 : ew - sw;
        m_c = (uint32_t)min<uint64_t>(a.chunk, a.n - c * a.chunk);
        const uint32_t sj = (uint32_t)(((uint64_t)j * wc) >> a.log2k) << 5;
        const uint32_t gj = gap_of(d.gaps, u);
        if (j == 0 && gj != 0) bad = true;
        start_bit = sj + gj;
        if (!last) {
            sj1 = (uint32_t)(((uint64_t)(j + 1) * wc) >> a.log2k) << 5;
            end_bit = sj1 + gap_of(d.gaps, u + 1);
            if (start_bit > end_bit) bad = true;
        } else {
            end_bit = wc ? (uint32_t)((wc - 1) << 5) : 0u;  // start of the last word
        }
    }

    Reader<NT> r;
    r.ring = &S.ring[0][tid];
    r.p = d.payload;
    r.sw = sw;
    r.gmax = d.payload_words ? (d.payload_words - 1) >> 2 : 0;
    r.sh = (uint32_t)sw & (RING - 1);
    const bool run = active && !bad;

    __syncthreads();  // tables complete

    // ---- 1. count
    uint32_t cnt = 0;
    if (run) {
        r.start(start_bit);
        uint32_t e = 0, inval = 0;
        // pos() < end_bit  <=>  off < thr = endq - 32 * rq
        const int32_t endq = (int32_t)(end_bit + 32 * (r.sh + 2));
        int32_t thr = endq - (int32_t)(r.rq << 5);
        // (a) far from the end: all code words that lie wholly inside the next
        // LUT_BITS bits at once, two such steps per refill; a step whose first
        // code word is longer decodes that one alone.  It stops while at least
        // 16 bits are left, so the last code word before `end` is decoded by
        // (b) and its length is known for the gap check.
        for (uint32_t it = 0; (int32_t)r.off + 2 * 16 + 16 <= thr; ++it) {
            if ((it & 3) == 0) r.tick();
            r.refill();
            thr = endq - (int32_t)(r.rq << 5);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t top = r.peek();
                const uint32_t m = T.mlut[top >> (32 - LUT_BITS)];
                if (m >= 16) {
                    r.off += m & 15u;
                    cnt += m >> 4;
                } else {
                    e = lookup(T, L, top, inval);
                    r.off += e & 0xFFu;
                    ++cnt;
                }
            }
        }
        // (b) the rest, one code word at a time, stopping exactly at `end`
        while ((int32_t)r.off < thr) {
            r.tick();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                r.refill();
                thr = endq - (int32_t)(r.rq << 5);
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    if ((int32_t)r.off < thr) {
                        e = step(T, L, r, inval);
                        ++cnt;
                    }
                }
            }
        }
        r.refill();
        bad |= inval != 0;
        if (!last) {
            const uint32_t pos = r.pos();
            if (pos != end_bit) bad = true;
            // the stored gap must name the FIRST code-word boundary at or after sj1
            if (cnt && end_bit != sj1 && pos - (e & 0xFFu) >= sj1) bad = true;
        }
    }

    // ---- 2. exclusive scan of counts within each chunk (segments of K lanes)
    // ring row 0 holds the counts now: a lane's column is its own, and no lane
    // touches the ring again before the barrier ahead of the decode pass
    uint32_t* const scnt = &S.ring[0][0];
    scnt[tid] = cnt;
    __syncthreads();
    for (int o = 1; o < DEC_THREADS; o <<= 1) {
        const uint32_t v = tid >= o ? scnt[tid - o] : 0u;
        __syncthreads();
        scnt[tid] += v;
        __syncthreads();
    }
    const int seg0 = tid - (int)j;  // lane of unit 0 of this chunk
    const uint32_t before_seg = seg0 > 0 ? scnt[seg0 - 1] : 0u;
    const uint32_t out_off = scnt[tid] - cnt - before_seg;
    uint64_t used_bits = 0;
    if (run && !bad) {
        if (last) {
            // the code words left in the chunk's last word, then zero padding
            if (out_off + cnt > m_c || m_c - out_off - cnt > 32) {
                bad = true;
            } else {
                // they lie in the last payload word, which the window holds
                // after the count pass (w0): no ring words are needed (the
                // ring's row 0 holds the counts)
                const uint32_t rem = m_c - out_off - cnt;
                uint32_t inval = 0;
                for (uint32_t i = 0; i < rem; ++i) {
                    r.refill();
                    (void)step(T, L, r, inval);
                }
                r.refill();
                cnt += rem;
                const uint32_t endw = (uint32_t)(wc << 5);
                const uint32_t pos = r.pos();
                if (inval || pos > endw || pos + 32 <= endw) {
                    bad = true;
                } else {
                    const uint32_t rest = endw - pos;
                    if (rest && (r.peek() >> (32 - rest)) != 0) bad = true;
                }
                used_bits = pos - start_bit;
            }
        } else {
            if (out_off + cnt > m_c) bad = true;
            used_bits = end_bit - start_bit;
        }
    }

    // padding bytes of the header are part of the format
    if (bid == 0) {
        for (uint64_t b = d.table_pad_from + tid; b < d.table_pad_to; b += DEC_THREADS)
            bad |= d.stream[b] != 0;
        for (uint64_t b = d.gap_pad_from + tid; b < d.gap_pad_to; b += DEC_THREADS)
            bad |= d.stream[b] != 0;
        if (tid == 0 && ((a.nc << a.log2k) & 1))
            bad |= (d.stream[d.gap_pad_from - 1] >> 4) != 0;
    }
    const int wg_bad = __syncthreads_or(bad);

    // ---- 3. decode pass: the DEC_BLOCK-byte blocks (aligned within the chunk's
    // output) that start in this lane's range; each goes out as whole 16-byte
    // stores, so every written sector of the output is written completely
    if (run && !wg_bad) {
        uint8_t* const base = d.out + c * a.chunk + out_off;
        const uint32_t h = (DEC_BLOCK - (out_off & (DEC_BLOCK - 1))) & (DEC_BLOCK - 1);
        const uint32_t nblk = cnt > h ? (cnt - h + DEC_BLOCK - 1) / DEC_BLOCK : 0u;
        if (nblk) {
            r.start(start_bit);
            uint32_t inval = 0;  // cannot be set: the count pass read the same bits
            for (uint32_t i = 0; i < h; ++i) {
                if ((i & 3) == 0) r.tick();
                r.refill();
                (void)step(T, L, r, inval);
            }
            uint8_t* dst = base + h;
            // blocks before the tensor end
            const uint32_t full = min(nblk, (m_c - out_off - h) / DEC_BLOCK);
            uint32_t b = 0;
            for (; b < full; ++b) {
                uint32_t w[DEC_BLOCK / 4];
                uint32_t ev[4];
#pragma unroll
                for (int q = 0; q < DEC_BLOCK / 2; ++q) {
                    if ((q & 3) == 0) r.tick();
                    r.refill();
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const int i = 2 * q + k;
                        ev[i & 3] = step(T, L, r, inval);
                        if ((i & 3) == 3) w[i >> 2] = syms4(ev);
                    }
                }
#pragma unroll
                for (int q = 0; q < DEC_BLOCK / 16; ++q) {
                    v4u v;
                    v.x = w[4 * q];
                    v.y = w[4 * q + 1];
                    v.z = w[4 * q + 2];
                    v.w = w[4 * q + 3];
                    *reinterpret_cast<v4u*>(dst + DEC_BLOCK * b + 16 * q) = v;
                }
            }
            if (b < nblk) {
                // the tensor ends inside this block: byte stores up to its end
                const uint32_t left = m_c - out_off - h - DEC_BLOCK * b;
                for (uint32_t i = 0; i < left; ++i) {
                    if ((i & 3) == 0) r.tick();
                    r.refill();
                    const uint32_t e = step(T, L, r, inval);
                    dst[DEC_BLOCK * b + i] = (uint8_t)(e >> 8);
                }
            }
        }
    }

    // ---- status, accounting, exit
    uint64_t v = used_bits;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if ((tid & 63) == 0) S.red[tid >> 6] = v;
    const int any_bad = __syncthreads_or(bad);
    if (tid == 0) {
        uint64_t tot = 0;
        for (int w = 0; w < DEC_THREADS / 64; ++w) tot += S.red[w];
        if (tot) atomicAdd(reinterpret_cast<unsigned long long*>(&d.ws->bits), (unsigned long long)tot);
        if (any_bad) atomicCAS(&d.ws->status, 0, (int32_t)LECB_ERR_CORRUPT);
        __threadfence();
        WsHeader* ws0 = a.st[0].ws;
        const uint32_t done = __hip_atomic_fetch_add(&ws0->exit_count, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            for (uint32_t k = 0; k < a.nstreams; ++k) {
                DecStream e = a.st[k];
                if (a.sizes) {
                    const uint64_t bytes = a.sizes[k].bytes;
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

}  // namespace

int launch_decode(const DecodeLaunch& L, void* stream) {
    DecArgs a{};
    const uint64_t tb = table_bytes(L.nc), gb = gap_bytes(L.nc, L.chunk);
    const uint32_t K = units_per_chunk(L.chunk);
    a.chunk = L.chunk;
    a.log2k = (uint32_t)ilog2(K);
    a.n = L.n;
    a.nc = L.nc;
    a.nstreams = L.nstreams;
    a.sizes = L.dev_sizes;
    for (int s = 0; s < L.nstreams; ++s) {
        DecStream& st = a.st[s];
        st.table = reinterpret_cast<const uint32_t*>(L.stream_base[s]);
        st.gaps = L.stream_base[s] + tb;
        st.payload = reinterpret_cast<const uint32_t*>(L.stream_base[s] + tb + gb);
        st.payload_words = L.dev_sizes ? 0 : (L.stream_bytes[s] - tb - gb) / 4;
        st.cb = L.cb[s];
        st.header_bytes = tb + gb;
        st.stream = L.stream_base[s];
        st.table_pad_from = 4 * L.nc;
        st.table_pad_to = tb;
        st.gap_pad_from = tb + (L.nc * K + 1) / 2;
        st.gap_pad_to = tb + gb;
        st.out = L.out[s];
        st.res = L.res[s];
        st.ws = L.ws[s];
    }
    const uint64_t units = L.nc * K;
    // Lanes per workgroup: the tables are one copy per workgroup, so bigger
    // workgroups leave more LDS for lanes (2 x 1024 lanes fit a CU against
    // 5 x 256), and fewer, bigger workgroups spread evenly over the CUs.
    // Take the biggest size that still gives every CU a workgroup.
    const uint64_t all = units * (uint64_t)L.nstreams;
    const uint64_t cus = (uint64_t)device_cu_count();
    const int nt = all >= cus * 1024 ? 1024 : all >= cus * 512 ? 512 : 256;
    a.wg_per_stream = (uint32_t)((units + nt - 1) / nt);
    const dim3 grid((uint32_t)((uint64_t)a.wg_per_stream * L.nstreams));
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (nt == 1024) hipLaunchKernelGGL(decode_kernel<1024>, grid, dim3(1024), 0, hs, a);
    else if (nt == 512) hipLaunchKernelGGL(decode_kernel<512>, grid, dim3(512), 0, hs, a);
    else hipLaunchKernelGGL(decode_kernel<256>, grid, dim3(256), 0, hs, a);
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

}  // namespace lecb
