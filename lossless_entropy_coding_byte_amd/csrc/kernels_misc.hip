// Histogram, byte-group split/merge (16- and 32-bit elements), fill.
//
// Histogram: "Single-Stage Huffman Encoder for ML Compression", Overview
// (frequency analysis) and Methodology step 1; "Lossless Compression for LLM
// Tensor Incremental Snapshots", Technical framework step 2.  Byte grouping:
// same page, Technical framework step 1 and the byte-group restore.
#include <hip/hip_runtime.h>

#include <atomic>

#include "lecb_internal.hpp"

namespace lecb {

namespace {

constexpr int HIST_THREADS = 256;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
__device__ inline v4u ld_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
}
__device__ inline void st_stream(void* p, v4u v) {
    __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(p));
}

// Each workgroup counts into LDS sub-histograms replicated R ways; lane l
// uses replica l % R and bin b of replica r sits at word b*R + r, so the 32
// lanes of a half-wave always hit 32 different banks whatever the data (a
// skewed plane such as a snapshot delta's high bytes is ~98 % one value).
template <int R>
__device__ inline void hist_add(uint32_t* s, uint32_t word, int r) {
    atomicAdd(&s[((word)&0xFFu) * R + r], 1u);
    atomicAdd(&s[((word >> 8) & 0xFFu) * R + r], 1u);
    atomicAdd(&s[((word >> 16) & 0xFFu) * R + r], 1u);
    atomicAdd(&s[(word >> 24) * R + r], 1u);
}

template <int R>
__device__ inline void hist_flush(const uint32_t* s, unsigned long long* out) {
    const int b = threadIdx.x;  // HIST_THREADS == 256 bins
    uint32_t sum = 0;
#pragma unroll
    for (int k = 0; k < R; ++k) sum += s[b * R + ((k + b) & (R - 1))];
    if (sum) atomicAdd(&out[b], (unsigned long long)sum);
}

__global__ __launch_bounds__(HIST_THREADS) void hist_u8_kernel(const uint8_t* __restrict__ in,
                                                               uint64_t n,
                                                               unsigned long long* hist) {
    constexpr int R = 32;
    __shared__ uint32_t s[256 * R];
    for (int i = threadIdx.x; i < 256 * R; i += HIST_THREADS) s[i] = 0;
    __syncthreads();
    const int r = threadIdx.x & (R - 1);
    const uint64_t n16 = n / 16;
    const uint4* in4 = reinterpret_cast<const uint4*>(in);
    const uint64_t stride = (uint64_t)gridDim.x * HIST_THREADS;
    // four 16-byte loads in flight per thread, then their 64 increments
    uint64_t i = (uint64_t)blockIdx.x * HIST_THREADS + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        v4u v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = ld_stream(&in4[i + q * stride]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            hist_add<R>(s, v[q].x, r);
            hist_add<R>(s, v[q].y, r);
            hist_add<R>(s, v[q].z, r);
            hist_add<R>(s, v[q].w, r);
        }
    }
    for (; i < n16; i += stride) {
        const v4u v = ld_stream(&in4[i]);
        hist_add<R>(s, v.x, r);
        hist_add<R>(s, v.y, r);
        hist_add<R>(s, v.z, r);
        hist_add<R>(s, v.w, r);
    }
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = n16 * 16 + threadIdx.x; i < n; i += HIST_THREADS)
            atomicAdd(&s[in[i] * R + r], 1u);
    }
    __syncthreads();
    hist_flush<R>(s, hist);
}

// in2 != nullptr: histograms of the planes of in[i] ^ in2[i] (snapshot delta)
__global__ __launch_bounds__(HIST_THREADS) void hist_u16_kernel(const uint16_t* __restrict__ in,
                                                                const uint16_t* __restrict__ in2,
                                                                uint64_t n,
                                                                unsigned long long* hist_hi,
                                                                unsigned long long* hist_lo) {
    // 32 replicas per plane (64 KiB of LDS): with 16, lanes l and l + 16 of a
    // half-wave shared a replica, and on a skewed plane they collided on the
    // same counter
    constexpr int R = 32;
    __shared__ uint32_t s_hi[256 * R];
    __shared__ uint32_t s_lo[256 * R];
    for (int i = threadIdx.x; i < 256 * R; i += HIST_THREADS) {
        s_hi[i] = 0;
        s_lo[i] = 0;
    }
    __syncthreads();
    const int r = threadIdx.x & (R - 1);
    const uint64_t n8 = n / 8;
    const uint4* in4 = reinterpret_cast<const uint4*>(in);
    const uint4* in24 = reinterpret_cast<const uint4*>(in2);
    const uint64_t stride = (uint64_t)gridDim.x * HIST_THREADS;
    auto add8 = [&](const v4u& v) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            atomicAdd(&s_lo[(w[k] & 0xFFu) * R + r], 1u);
            atomicAdd(&s_hi[((w[k] >> 8) & 0xFFu) * R + r], 1u);
            atomicAdd(&s_lo[((w[k] >> 16) & 0xFFu) * R + r], 1u);
            atomicAdd(&s_hi[(w[k] >> 24) * R + r], 1u);
        }
    };
    // eight 16-byte loads in flight per thread, then their 128 increments
    uint64_t i = (uint64_t)blockIdx.x * HIST_THREADS + threadIdx.x;
    for (; i + 7 * stride < n8; i += 8 * stride) {
        v4u v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = ld_stream(&in4[i + q * stride]);
        if (in2) {
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] ^= ld_stream(&in24[i + q * stride]);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) add8(v[q]);
    }
    for (; i < n8; i += stride) add8(in2 ? ld_stream(&in4[i]) ^ ld_stream(&in24[i]) : ld_stream(&in4[i]));
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = n8 * 8 + threadIdx.x; i < n; i += HIST_THREADS) {
            const uint32_t x = in2 ? (uint32_t)(in[i] ^ in2[i]) : in[i];
            atomicAdd(&s_lo[(x & 0xFFu) * R + r], 1u);
            atomicAdd(&s_hi[(x >> 8) * R + r], 1u);
        }
    }
    __syncthreads();
    hist_flush<R>(s_hi, hist_hi);
    hist_flush<R>(s_lo, hist_lo);
}

// Four byte planes of 32-bit elements; s[p] counts byte 3 - p (most
// significant plane first), 16 replicas per plane (64 KiB of LDS).
__global__ __launch_bounds__(HIST_THREADS) void hist_u32_kernel(const uint32_t* __restrict__ in,
                                                                uint64_t n,
                                                                unsigned long long* hist) {
    constexpr int R = 16;
    __shared__ uint32_t s[4][256 * R];
    for (int i = threadIdx.x; i < 256 * R; i += HIST_THREADS) {
        s[0][i] = 0;
        s[1][i] = 0;
        s[2][i] = 0;
        s[3][i] = 0;
    }
    __syncthreads();
    const int r = threadIdx.x & (R - 1);
    const uint64_t n4 = n / 4;
    const uint4* in4 = reinterpret_cast<const uint4*>(in);
    const uint64_t stride = (uint64_t)gridDim.x * HIST_THREADS;
    auto add1 = [&](uint32_t x) {
        atomicAdd(&s[3][(x & 0xFFu) * R + r], 1u);
        atomicAdd(&s[2][((x >> 8) & 0xFFu) * R + r], 1u);
        atomicAdd(&s[1][((x >> 16) & 0xFFu) * R + r], 1u);
        atomicAdd(&s[0][(x >> 24) * R + r], 1u);
    };
    // four 16-byte loads in flight per thread, then their 64 increments
    uint64_t i = (uint64_t)blockIdx.x * HIST_THREADS + threadIdx.x;
    for (; i + 3 * stride < n4; i += 4 * stride) {
        v4u v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = ld_stream(&in4[i + q * stride]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            add1(v[q].x);
            add1(v[q].y);
            add1(v[q].z);
            add1(v[q].w);
        }
    }
    for (; i < n4; i += stride) {
        const v4u v = ld_stream(&in4[i]);
        add1(v.x);
        add1(v.y);
        add1(v.z);
        add1(v.w);
    }
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = n4 * 4 + threadIdx.x; i < n; i += HIST_THREADS) add1(in[i]);
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) hist_flush<R>(s[p], hist + 256 * p);
}

constexpr int BG_THREADS = 256;

// 16 elements per thread: two 16-byte loads of u16, two 16-byte stores.
__device__ inline uint32_t pick_lo(uint32_t a, uint32_t b) {
    return (a & 0xFFu) | ((a >> 8) & 0xFF00u) | ((b & 0xFFu) << 16) | ((b << 8) & 0xFF000000u);
}
__device__ inline uint32_t pick_hi(uint32_t a, uint32_t b) {
    return ((a >> 8) & 0xFFu) | ((a >> 16) & 0xFF00u) | ((b << 8) & 0xFF0000u) | (b & 0xFF000000u);
}

__global__ __launch_bounds__(BG_THREADS) void split_kernel(const uint16_t* __restrict__ in,
                                                           uint64_t n, uint8_t* __restrict__ hi,
                                                           uint8_t* __restrict__ lo) {
    const uint64_t n16 = n / 16;
    const uint64_t stride = (uint64_t)gridDim.x * BG_THREADS;
    for (uint64_t i = (uint64_t)blockIdx.x * BG_THREADS + threadIdx.x; i < n16; i += stride) {
        const v4u a = ld_stream(reinterpret_cast<const uint4*>(in) + 2 * i);
        const v4u b = ld_stream(reinterpret_cast<const uint4*>(in) + 2 * i + 1);
        v4u h, l;
        l.x = pick_lo(a.x, a.y); l.y = pick_lo(a.z, a.w); l.z = pick_lo(b.x, b.y); l.w = pick_lo(b.z, b.w);
        h.x = pick_hi(a.x, a.y); h.y = pick_hi(a.z, a.w); h.z = pick_hi(b.x, b.y); h.w = pick_hi(b.z, b.w);
        st_stream(reinterpret_cast<uint4*>(hi) + i, h);
        st_stream(reinterpret_cast<uint4*>(lo) + i, l);
    }
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = n16 * 16 + threadIdx.x; i < n; i += BG_THREADS) {
            hi[i] = (uint8_t)(in[i] >> 8);
            lo[i] = (uint8_t)(in[i] & 0xFF);
        }
    }
}

// Restores: every lane writes 16 consecutive output bytes per store, and the
// lanes of a wave write consecutive 16-byte pieces, so each store instruction
// covers whole cache lines (no partly written lines reach HBM).

// Elements 2*half, 2*half+1 from the high and low byte words h, l.
__device__ inline uint32_t join2(uint32_t h, uint32_t l, int half) {
    const uint32_t hs = half ? (h >> 16) : h;
    const uint32_t ls = half ? (l >> 16) : l;
    return (ls & 0xFFu) | ((hs & 0xFFu) << 8) | ((ls & 0xFF00u) << 8) | ((hs & 0xFF00u) << 16);
}

typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// 8 elements per lane and step: 8 bytes of each plane in, 16 bytes out.
// w0 != nullptr: out = w0 ^ (hi << 8 | lo) (a snapshot from its delta)
__global__ __launch_bounds__(BG_THREADS) void merge_kernel(const uint8_t* __restrict__ hi,
                                                           const uint8_t* __restrict__ lo,
                                                           const uint16_t* __restrict__ w0,
                                                           uint64_t n, uint16_t* __restrict__ out) {
    const uint64_t n8 = n / 8;
    const uint64_t stride = (uint64_t)gridDim.x * BG_THREADS;
    for (uint64_t i = (uint64_t)blockIdx.x * BG_THREADS + threadIdx.x; i < n8; i += stride) {
        const v2u h = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(hi) + i);
        const v2u l = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(lo) + i);
        v4u a;
        a.x = join2(h.x, l.x, 0);
        a.y = join2(h.x, l.x, 1);
        a.z = join2(h.y, l.y, 0);
        a.w = join2(h.y, l.y, 1);
        if (w0) a ^= ld_stream(reinterpret_cast<const uint4*>(w0) + i);
        st_stream(reinterpret_cast<uint4*>(out) + i, a);
    }
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = n8 * 8 + threadIdx.x; i < n; i += BG_THREADS)
            out[i] = (uint16_t)((((uint16_t)hi[i] << 8) | lo[i]) ^ (w0 ? w0[i] : 0));
    }
}

// Byte k of the four plane words, as one 32-bit element (planes 3..0).
__device__ inline uint32_t join4(uint32_t w3, uint32_t w2, uint32_t w1, uint32_t w0, int k) {
    const int sh = 8 * k;
    return ((w0 >> sh) & 0xFFu) | (((w1 >> sh) & 0xFFu) << 8) | (((w2 >> sh) & 0xFFu) << 16) |
           (((w3 >> sh) & 0xFFu) << 24);
}

// 4 elements per lane and step: 4 bytes of each plane in, 16 bytes out.
__global__ __launch_bounds__(BG_THREADS) void merge4_kernel(const uint8_t* __restrict__ p3,
                                                            const uint8_t* __restrict__ p2,
                                                            const uint8_t* __restrict__ p1,
                                                            const uint8_t* __restrict__ p0, uint64_t n,
                                                            uint32_t* __restrict__ out) {
    const uint64_t n4 = n / 4;
    const uint64_t stride = (uint64_t)gridDim.x * BG_THREADS;
    for (uint64_t i = (uint64_t)blockIdx.x * BG_THREADS + threadIdx.x; i < n4; i += stride) {
        const uint32_t w3 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p3) + i);
        const uint32_t w2 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p2) + i);
        const uint32_t w1 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p1) + i);
        const uint32_t w0 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p0) + i);
        v4u o;
        o.x = join4(w3, w2, w1, w0, 0);
        o.y = join4(w3, w2, w1, w0, 1);
        o.z = join4(w3, w2, w1, w0, 2);
        o.w = join4(w3, w2, w1, w0, 3);
        st_stream(reinterpret_cast<uint4*>(out) + i, o);
    }
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = n4 * 4 + threadIdx.x; i < n; i += BG_THREADS)
            out[i] = ((uint32_t)p3[i] << 24) | ((uint32_t)p2[i] << 16) | ((uint32_t)p1[i] << 8) | p0[i];
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint8_t* p, uint64_t bytes) {
    const uint64_t n16 = bytes / 16;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    const uint4 z = {0, 0, 0, 0};
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        reinterpret_cast<uint4*>(p)[i] = z;
    if (blockIdx.x == 0)
        for (uint64_t i = n16 * 16 + threadIdx.x; i < bytes; i += blockDim.x) p[i] = 0;
}

__global__ void result_kernel(lecb_result* r, uint64_t bytes, uint64_t bits, int32_t status) {
    r->bytes = bytes;
    r->payload_bits = bits;
    r->status = status;
    r->reserved = 0;
}

int grid_for(uint64_t items, int threads, int max_blocks) {
    uint64_t g = (items + threads - 1) / threads;
    if (g < 1) g = 1;
    if (g > (uint64_t)max_blocks) g = max_blocks;
    return (int)g;
}

}  // namespace

int device_cu_count() {
    // per device, asked once; concurrent first calls store the same value
    static std::atomic<int> cached[MAX_DEVICES];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return 256;
    int cus = cached[dev].load(std::memory_order_relaxed);
    if (!cus) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

int launch_histogram_u8(const uint8_t* in, uint64_t n, uint64_t* hist, int accumulate,
                        void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!accumulate) {
        int rc = launch_fill_zero(hist, 256 * sizeof(uint64_t), stream);
        if (rc) return rc;
    }
    if (n == 0) return LECB_OK;
    // one workgroup per compute unit: fewer flushes of the 256 bins into the
    // same global counters (measured best for this kernel)
    const int grid = grid_for(n / 16 + 1, HIST_THREADS * 8, device_cu_count());
    hipLaunchKernelGGL(hist_u8_kernel, dim3(grid), dim3(HIST_THREADS), 0, s, in, n,
                       reinterpret_cast<unsigned long long*>(hist));
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

int launch_histogram_u16(const uint16_t* in, const uint16_t* in2, uint64_t n, uint64_t* hist_hi,
                         uint64_t* hist_lo, int accumulate, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!accumulate) {
        // one fill when the two histograms are adjacent (the usual layout)
        int rc;
        if (hist_lo == hist_hi + 256) {
            rc = launch_fill_zero(hist_hi, 512 * sizeof(uint64_t), stream);
        } else {
            rc = launch_fill_zero(hist_hi, 256 * sizeof(uint64_t), stream);
            if (!rc) rc = launch_fill_zero(hist_lo, 256 * sizeof(uint64_t), stream);
        }
        if (rc) return rc;
    }
    if (n == 0) return LECB_OK;
    // two workgroups per compute unit (measured best: fewer global flushes)
    const int grid = grid_for(n / 8 + 1, HIST_THREADS * 8, device_cu_count() * 2);
    hipLaunchKernelGGL(hist_u16_kernel, dim3(grid), dim3(HIST_THREADS), 0, s, in, in2, n,
                       reinterpret_cast<unsigned long long*>(hist_hi),
                       reinterpret_cast<unsigned long long*>(hist_lo));
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

int launch_histogram_u32(const uint32_t* in, uint64_t n, uint64_t* hist, int accumulate, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!accumulate) {
        const int rc = launch_fill_zero(hist, 4 * 256 * sizeof(uint64_t), stream);
        if (rc) return rc;
    }
    if (n == 0) return LECB_OK;
    const int grid = grid_for(n / 4 + 1, HIST_THREADS * 8, device_cu_count() * 2);
    hipLaunchKernelGGL(hist_u32_kernel, dim3(grid), dim3(HIST_THREADS), 0, s, in, n,
                       reinterpret_cast<unsigned long long*>(hist));
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

int launch_merge4(const uint8_t* p3, const uint8_t* p2, const uint8_t* p1, const uint8_t* p0, uint64_t n,
                  uint32_t* out, void* stream) {
    if (n == 0) return LECB_OK;
    const int grid = grid_for(n / 4 + 1, BG_THREADS, device_cu_count() * 16);
    hipLaunchKernelGGL(merge4_kernel, dim3(grid), dim3(BG_THREADS), 0,
                       reinterpret_cast<hipStream_t>(stream), p3, p2, p1, p0, n, out);
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

int launch_split(const uint16_t* in, uint64_t n, uint8_t* hi, uint8_t* lo, void* stream) {
    if (n == 0) return LECB_OK;
    const int grid = grid_for(n / 16 + 1, BG_THREADS, device_cu_count() * 16);
    hipLaunchKernelGGL(split_kernel, dim3(grid), dim3(BG_THREADS), 0,
                       reinterpret_cast<hipStream_t>(stream), in, n, hi, lo);
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

int launch_merge(const uint8_t* hi, const uint8_t* lo, const uint16_t* w0, uint64_t n, uint16_t* out,
                 void* stream) {
    if (n == 0) return LECB_OK;
    const int grid = grid_for(n / 8 + 1, BG_THREADS, device_cu_count() * 16);
    hipLaunchKernelGGL(merge_kernel, dim3(grid), dim3(BG_THREADS), 0,
                       reinterpret_cast<hipStream_t>(stream), hi, lo, w0, n, out);
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

int launch_result(lecb_result* r, uint64_t bytes, uint64_t bits, int32_t status, void* stream) {
    hipLaunchKernelGGL(result_kernel, dim3(1), dim3(1), 0, reinterpret_cast<hipStream_t>(stream), r,
                       bytes, bits, status);
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

int launch_fill_zero(void* ptr, uint64_t bytes, void* stream) {
    if (bytes == 0) return LECB_OK;
    const int grid = grid_for(bytes / 16 + 1, 256, device_cu_count() * 8);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<uint8_t*>(ptr),
                       bytes);
    return hipGetLastError() == hipSuccess ? LECB_OK : LECB_ERR_HIP;
}

}  // namespace lecb
