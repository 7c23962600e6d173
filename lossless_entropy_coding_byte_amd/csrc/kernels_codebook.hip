// Device codebooks: the decode and encode tables from a canonical
// description, and the whole per-tensor codebook built on the device.
//
// "Single-Stage Huffman Encoder for ML Compression", Methodology step 3 (the
// codebook is stored on each accelerator) and Overview (classic per-shard
// Huffman coding: frequency analysis, codebook generation, codebook
// transmission); "Lossless Compression for LLM Tensor Incremental
// Snapshots", Technical framework step 3 and Key design item 2 (an efficient
// Huffman-tree build).
//
// build_kernel: one workgroup per histogram computes the optimal code
// lengths under the length limit with package-merge (Larmore & Hirschberg),
// then the canonical code words, with the tie rule of the host builder:
// coins ordered by (frequency, byte value), a coin ahead of a package of the
// same weight.  Each level's merged list is formed in parallel: coin i lands
// at i + (packages lighter than it), package j at j + (coins not heavier than
// it), both found by binary search in the sorted lists.  A coin's code length
// is the number of levels whose selected prefix holds it; the selected
// prefixes come from counting the packages in the prefix, level by level from
// the top.
#include <hip/hip_runtime.h>

#include "lecb_internal.hpp"

namespace lecb {

namespace {

constexpr int CB_THREADS = 256;

// Length of the code word that the left-aligned 16-bit window w starts with:
// the windows of length-l code words are [limit[l-1], limit[l]), so it is 1 +
// the number of limits at or below w (17: no code word starts at w).
__device__ inline uint32_t code_len(const uint32_t* limit, uint32_t w) {
    uint32_t n = 1;
#pragma unroll
    for (int l = 1; l <= 16; ++l) n += w >= limit[l];
    return n;
}

// Entry i of the decode table (see DeviceCodebook::dec).
__device__ inline uint16_t dec_entry(const uint32_t* limit, const uint32_t* first, const uint32_t* base,
                                     const uint8_t* sorted, uint32_t i) {
    const uint32_t lb = limit[LUT_BITS], b4 = lb >> 4;
    if (i < b4) {
        // a code word of at most LUT_BITS bits starts every window below lb
        const uint32_t l = code_len(limit, i << (16 - LUT_BITS));
        return (uint16_t)((sorted[(base[l] + (i >> (LUT_BITS - l)) - first[l]) & 255u] << 8) | l);
    }
    const uint32_t v = lb + (i - b4);
    if (i >= (uint32_t)DEC_SIZE || v >= limit[16]) return DEC_INVALID;
    const uint32_t l = code_len(limit, v);
    return (uint16_t)((sorted[(base[l] + (v >> (16 - l)) - first[l]) & 255u] << 8) | l);
}

__device__ inline void long_fields(const uint32_t* limit, DeviceCodebook* cb) {
    cb->long_base = limit[LUT_BITS];
    cb->long_sub = limit[LUT_BITS] - (limit[LUT_BITS] >> 4);
    cb->pad[0] = 0;
}

// Tables from the canonical description passed by value (host-built codebook).
// Grid covers the DEC_ENTRIES decode table entries.
__global__ __launch_bounds__(CB_THREADS) void codebook_kernel(CodebookArgs a, DeviceCodebook* cb) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < 256) {
        cb->enc[t] = a.enc[t];
        cb->sorted[t] = a.sorted[t];
    }
    if (t < 17) {
        cb->first[t] = a.first[t];
        cb->base[t] = a.base[t];
        cb->limit[t] = t ? (a.first[t] + a.count[t]) << (16 - t) : 0;
    }
    if (t == 0) {
        cb->max_len = a.max_len;
        cb->num_coded = a.num_coded;
    }
    uint32_t limit[17];
    limit[0] = 0;
    for (int l = 1; l <= 16; ++l) limit[l] = (a.first[l] + a.count[l]) << (16 - l);
    if (t == 0) long_fields(limit, cb);
    if (t < DEC_ENTRIES) cb->dec[t] = dec_entry(limit, a.first, a.base, a.sorted, (uint32_t)t);
}

struct BuildArgs {
    const uint64_t* hist[4];
    DeviceCodebook* cb[4];
    uint32_t max_len;
    uint32_t min_freq;
};

// One workgroup per histogram: lengths, canonical code words, enc / first /
// base / limit / sorted of the device codebook.  No codebook (histogram empty
// after the clamp, or more coded symbols than 2^max_len): every length 0.
// The coins are ordered by a bitonic sort, the two binary searches of a level
// run in the same loop, and the canonical ranks come from wave ballots, so the
// work is a few hundred dependent LDS latencies in all.
__global__ __launch_bounds__(CB_THREADS) void build_kernel(BuildArgs a) {
    __shared__ uint64_t f[256];        // clamped frequency per byte value
    __shared__ uint64_t coin[257];     // coded symbols' weights by (frequency, byte value)
    __shared__ uint8_t order[256];     // byte value of coin i
    __shared__ uint64_t lst[2][512];   // merged lists of two consecutive levels
    __shared__ uint32_t pkg[16][16];   // which items of level k's list are packages
    __shared__ uint32_t pre[16][16];   // packages in words 0..w-1 of level k's bits
    __shared__ uint32_t len_at[16], coins_at[16];
    __shared__ __attribute__((aligned(16))) uint8_t len[256];
    __shared__ uint32_t count[17], first[17], base[17];
    __shared__ uint32_t fail, maxl;
    __shared__ uint64_t lmask[17][4];

    const int tid = threadIdx.x;
    const int L = (int)a.max_len;
    const int plane = blockIdx.x;
    uint64_t fs = a.hist[plane][tid];
    fs = fs > a.min_freq ? fs : (uint64_t)a.min_freq;
    f[tid] = fs;
    order[tid] = (uint8_t)tid;
    len[tid] = 0;
    pkg[tid >> 4][tid & 15] = 0;
    if (tid <= 16) count[tid] = 0;
    if (tid == 0) {
        fail = 0;
        maxl = 0;
        coin[256] = 0;
    }
    const bool coded = fs > 0;
    const int m = __syncthreads_count(coded);
    {
        // bitonic sort of (frequency, byte value) ascending; the 256 - m
        // uncoded values (frequency 0) come first, coin i sits at 256 - m + i
        uint64_t kf = fs;
        uint32_t ks = (uint32_t)tid;
        for (int k = 2; k <= 256; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                const int q = tid ^ j;
                const uint64_t pf = f[q];
                const uint32_t ps = order[q];
                const bool mine_less = kf < pf || (kf == pf && ks < ps);
                // ascending block when (tid & k) == 0: the lower index keeps the smaller
                const bool keep_small = ((tid & k) == 0) == (tid < q);
                if (keep_small != mine_less) {
                    kf = pf;
                    ks = ps;
                }
                __syncthreads();
                f[tid] = kf;
                order[tid] = (uint8_t)ks;
                __syncthreads();
            }
        }
        if (tid >= 256 - m) coin[tid - (256 - m)] = kf;
        __syncthreads();
        // order[] now holds byte values in sorted order from index 256 - m on
        const uint8_t sym = order[tid];
        __syncthreads();
        if (tid >= 256 - m) order[tid - (256 - m)] = sym;
    }
    __syncthreads();
    if (m >= 2 && (uint64_t)m <= (1ull << L)) {
        if (tid < m) lst[0][tid] = coin[tid];
        if (tid == 0) len_at[0] = m;
        int cur = 0, cur_n = m;
        __syncthreads();
        for (int k = 1; k < L; ++k) {
            const int np = cur_n / 2;
            const uint64_t* c = lst[cur];
            uint64_t* nx = lst[cur ^ 1];
            // coin tid: the packages lighter than it (first j with weight >= it);
            // package tid: the coins not heavier than it (first i heavier)
            const bool hc = tid < m, hp = tid < np;
            const uint64_t cw = coin[tid];
            const uint64_t pw = hp ? c[2 * tid] + c[2 * tid + 1] : 0;
            int clo = 0, chi = hc ? np : 0, plo = 0, phi = hp ? m : 0;
            const int nit = 32 - __clz((uint32_t)max(m, np));  // halvings to empty either range
#pragma unroll
            for (int it = 0; it < 9; ++it) {  // nit <= 9 (m <= 256)
                if (it >= nit) break;
                const int cm = (clo + chi) >> 1, pm = (plo + phi) >> 1;
                const uint64_t a0 = c[2 * cm], a1 = c[2 * cm + 1];  // 2*cm+1 <= cur_n < 512
                const uint64_t b = coin[pm];                        // pm <= 256
                if (clo < chi) {
                    if (a0 + a1 < cw) clo = cm + 1;
                    else chi = cm;
                }
                if (plo < phi) {
                    if (b <= pw) plo = pm + 1;
                    else phi = pm;
                }
            }
            if (hc) nx[tid + clo] = cw;
            if (hp) {
                const int pos = tid + plo;
                nx[pos] = pw;
                atomicOr(&pkg[k][pos >> 5], 1u << (pos & 31));
            }
            const int nn = m + np;
            if (tid == 0) len_at[k] = nn;
            __syncthreads();
            // a level equal to the one before repeats up to the top: stop here
            bool diff = nn != cur_n;
            if (!diff) {
                diff = (tid < nn && nx[tid] != c[tid]) || (tid + 256 < nn && nx[tid + 256] != c[tid + 256]);
                if (tid < 16) diff |= pkg[k][tid] != pkg[k - 1][tid];
            }
            cur_n = nn;
            cur ^= 1;
            if (!__syncthreads_or(diff)) {
                for (int q = tid; q < (L - 1 - k) * 16; q += CB_THREADS) pkg[k + 1 + q / 16][q & 15] = pkg[k][q & 15];
                if (tid < L - 1 - k) len_at[k + 1 + tid] = nn;
                __syncthreads();
                break;
            }
        }
        {
            // per level, the packages in the words before each word
            const int k = tid >> 4, w = tid & 15;
            const uint32_t cnt = __popc(pkg[k][w]);
            uint32_t incl = cnt;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const uint32_t t = __shfl_up(incl, o, 16);
                if (w >= o) incl += t;
            }
            pre[k][w] = incl - cnt;
        }
        __syncthreads();
        if (tid == 0) {
            // the top level's first 2m - 2 items; each package taken at level
            // k takes the two items it was made of at level k - 1
            uint32_t take = 2 * m - 2;
            for (int k = L - 1; k >= 0; --k) {
                if (take > len_at[k]) {
                    fail = 1;
                    break;
                }
                const uint32_t w = take >> 5, b = take & 31u;  // take <= 511
                const uint32_t np = pre[k][w] + (b ? __popc(pkg[k][w] & ((1u << b) - 1u)) : 0u);
                coins_at[k] = take - np;
                take = 2 * np;
            }
        }
        __syncthreads();
        if (tid < m && !fail) {
            uint32_t l = 0;
            for (int k = 0; k < L; ++k) l += (uint32_t)tid < coins_at[k];
            len[order[tid]] = (uint8_t)l;
        }
    } else if (m == 1 && tid == 0) {
        len[order[0]] = 1;
    }
    __syncthreads();

    // canonical code words: by length, then byte value
    const uint32_t ls = len[tid];
    if (ls) {
        atomicAdd(&count[ls], 1u);
        atomicMax(&maxl, ls);
    }
    const int ncoded = __syncthreads_count(ls != 0);
    if (tid == 0) {
        uint32_t code = 0, idx = 0;
        first[0] = 0;
        base[0] = 0;
        for (int l = 1; l <= 16; ++l) {
            code = (code + count[l - 1]) << 1;
            first[l] = code;
            base[l] = idx;
            idx += count[l];
        }
    }
    __syncthreads();
    // rank among the coded symbols of the same length with a smaller byte
    // value: per length and wave, the mask of lanes holding that length
    const int lane = tid & 63, wv = tid >> 6;
    for (int l = 1; l <= 16; ++l) {
        const uint64_t mk = __ballot(ls == (uint32_t)l);
        if (lane == 0) lmask[l][wv] = mk;
    }
    __syncthreads();
    uint32_t rank = 0;
    if (ls) {
        for (int w = 0; w < wv; ++w) rank += __popcll(lmask[ls][w]);
        rank += __popcll(lmask[ls][wv] & ((1ull << lane) - 1ull));
    }
    DeviceCodebook* cb = a.cb[plane];
    cb->enc[tid] = ls ? ((first[ls] + rank) << 5) | ls : 0u;
    if (ls) cb->sorted[base[ls] + rank] = (uint8_t)tid;
    if (tid >= ncoded) cb->sorted[tid] = 0;
    if (tid <= 16) {
        cb->first[tid] = first[tid];
        cb->base[tid] = base[tid];
        cb->limit[tid] = tid ? (first[tid] + count[tid]) << (16 - tid) : 0;
    }
    if (tid == 0) {
        cb->max_len = maxl;
        cb->num_coded = (uint32_t)ncoded;
    }
}

// Decode tables of device codebooks whose canonical description build_kernel
// wrote; grid (DEC_ENTRIES / 256 rounded up, codebooks).
__global__ __launch_bounds__(CB_THREADS) void tables_kernel(BuildArgs a) {
    __shared__ uint32_t first[17], base[17], lim[17];
    __shared__ uint8_t sorted[256];
    DeviceCodebook* cb = a.cb[blockIdx.y];
    const int tid = threadIdx.x;
    if (tid <= 16) {
        first[tid] = cb->first[tid];
        base[tid] = cb->base[tid];
        lim[tid] = cb->limit[tid];
    }
    sorted[tid] = cb->sorted[tid];
    __syncthreads();
    const uint32_t t = blockIdx.x * CB_THREADS + tid;
    if (t < (uint32_t)DEC_ENTRIES) cb->dec[t] = dec_entry(lim, first, base, sorted, t);
    if (t == 0) long_fields(lim, cb);
}

}  // namespace

int launch_codebook_upload(const CodebookArgs& args, DeviceCodebook* blob, void* stream) {
    hipLaunchKernelGGL(codebook_kernel, dim3((DEC_ENTRIES + CB_THREADS - 1) / CB_THREADS), dim3(CB_THREADS), 0,
                       reinterpret_cast<hipStream_t>(stream), args, blob);
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

int launch_build_codebooks(const uint64_t* const* hist, DeviceCodebook* const* cb, int n, uint32_t max_len,
                           uint32_t min_freq, void* stream) {
    if (n < 1 || n > 4) return LECB_ERR_INVALID_ARG;
    BuildArgs a{};
    for (int k = 0; k < n; ++k) {
        a.hist[k] = hist[k];
        a.cb[k] = cb[k];
    }
    a.max_len = max_len;
    a.min_freq = min_freq;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(build_kernel, dim3(n), dim3(CB_THREADS), 0, s, a);
    hipLaunchKernelGGL(tables_kernel, dim3((DEC_ENTRIES + CB_THREADS - 1) / CB_THREADS, n), dim3(CB_THREADS), 0, s, a);
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

}  // namespace lecb
