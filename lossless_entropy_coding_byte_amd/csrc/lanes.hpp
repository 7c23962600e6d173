// Lane geometry of stream format v3 and the wave-level helpers the encoder
// and the decoder share.
//
// A chunk is coded as G = min(chunk/256, 16) lanes; 16-symbol block b of the
// chunk belongs to lane b mod G.  On the GPU one hardware lane runs one coder
// lane, and a wave of 64 is four rows of 16: row r holds plane r % P (P byte
// planes handled together) of the 16/G chunks of row group r / P, lane i of
// the row being lane i mod G of chunk i / G of that row group.  The G lanes
// of a chunk therefore sit side by side inside one row, which is what the
// DPP broadcasts below rely on.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "lecb_internal.hpp"

namespace lecb {

constexpr uint32_t BLOCK = 16;   // symbols per block

// Where hardware lane `lane` (0..63) of a wave sits for P planes and chunks of
// G = 1 << LG lanes.
struct LanePlace {
    uint32_t plane;    // r % P
    uint32_t chunk;    // chunk index within the wave's task (row group major)
    uint32_t j;        // lane of that chunk
};

template <int P, int LG>
__device__ inline LanePlace lane_place(uint32_t lane) {
    const uint32_t r = lane >> 4, i = lane & 15u;
    LanePlace p;
    p.plane = r % P;
    p.chunk = (r / P) * (16u >> LG) + (i >> LG);
    p.j = i & ((1u << LG) - 1);
    return p;
}

// Chunks of one wave's task.
template <int P, int LG>
constexpr uint32_t chunks_per_task() { return (4 / P) * (16u >> LG); }

// Symbols of lane j of a chunk of m symbols (m <= chunk; S = chunk / G for a whole chunk).
template <int LG>
__device__ inline uint32_t lane_symbols(uint32_t m, uint32_t j) {
    constexpr uint32_t G = 1u << LG;
    const uint32_t full = m / BLOCK, rest = m % BLOCK;
    const uint32_t whole = full > j ? (full - j + G - 1) >> LG : 0u;
    return whole * BLOCK + ((full & (G - 1)) == j && rest ? rest : 0u);
}

// Value of lane `src` of the caller's row, broadcast over the row (DPP).
template <int SRC>
__device__ inline uint32_t row_bcast(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x150 + SRC, 0xF, 0xF, false);
}

// Exclusive count over the lanes of the caller's group (G = 1 << LG lanes,
// aligned inside a row) of the lanes whose bit of the wave mask `m` is set,
// and the group's total.  Every lane of the wave must call it (the broadcasts
// read neighbouring lanes).
template <int LG>
__device__ inline void group_count_mask(uint64_t m, uint32_t& before, uint32_t& total) {
    const uint32_t p = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    // inclusive count: p plus this lane's bit of m, taken as the carry-in
    uint32_t q;
    uint64_t carry_out;
    asm("v_addc_co_u32_e64 %0, %1, %2, 0, %3" : "=v"(q), "=s"(carry_out) : "v"(p), "s"(m));
    (void)carry_out;
    uint32_t first, last;
    if constexpr (LG == 0) {
        first = p;
        last = q;
    } else if constexpr (LG == 1) {
        first = (uint32_t)__builtin_amdgcn_mov_dpp((int)p, 0xA0, 0xF, 0xF, false);   // quad_perm [0,0,2,2]
        last = (uint32_t)__builtin_amdgcn_mov_dpp((int)q, 0xF5, 0xF, 0xF, false);    // quad_perm [1,1,3,3]
    } else if constexpr (LG == 2) {
        first = (uint32_t)__builtin_amdgcn_mov_dpp((int)p, 0x00, 0xF, 0xF, false);   // quad_perm [0,0,0,0]
        last = (uint32_t)__builtin_amdgcn_mov_dpp((int)q, 0xFF, 0xF, 0xF, false);    // quad_perm [3,3,3,3]
    } else if constexpr (LG == 3) {
        const bool hi = (threadIdx.x & 8u) != 0;
        const uint32_t f0 = row_bcast<0>(p), f8 = row_bcast<8>(p);
        const uint32_t l7 = row_bcast<7>(q), l15 = row_bcast<15>(q);
        first = hi ? f8 : f0;
        last = hi ? l15 : l7;
    } else {
        first = row_bcast<0>(p);
        last = row_bcast<15>(q);
    }
    before = p - first;
    total = last - first;
}

// The same for a per-lane flag `f` (its ballot is the mask).
template <int LG>
__device__ inline void group_count(bool f, uint32_t& before, uint32_t& total) {
    group_count_mask<LG>(__builtin_amdgcn_ballot_w64(f), before, total);
}

// Value of lane (lane ^ O) for O < 32: ds_swizzle in its bit mode (and mask
// 0x1F, or mask 0, xor mask O), the pattern an immediate, so no lane index
// stays in a register.
template <int O>
__device__ inline uint32_t lane_xor(uint32_t v) {
    static_assert(O > 0 && O < 32, "the swizzle works inside groups of 32 lanes");
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (O << 10));
}

// Maximum and minimum of v over the wave (wave-uniform): swizzles inside each
// half of 32 lanes, then the two halves' results read as scalars.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
    v = max(v, lane_xor<1>(v));
    v = max(v, lane_xor<2>(v));
    v = max(v, lane_xor<4>(v));
    v = max(v, lane_xor<8>(v));
    v = max(v, lane_xor<16>(v));
    return max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
}
__device__ inline uint32_t wave_min_u32(uint32_t v) {
    v = min(v, lane_xor<1>(v));
    v = min(v, lane_xor<2>(v));
    v = min(v, lane_xor<4>(v));
    v = min(v, lane_xor<8>(v));
    v = min(v, lane_xor<16>(v));
    return min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
}

// Sum of v over the caller's group of G = 1 << LG lanes (every lane gets it).
template <int LG>
__device__ inline uint32_t group_sum(uint32_t v) {
    if constexpr (LG >= 1) v += lane_xor<1>(v);
    if constexpr (LG >= 2) v += lane_xor<2>(v);
    if constexpr (LG >= 3) v += lane_xor<4>(v);
    if constexpr (LG >= 4) v += lane_xor<8>(v);
    return v;
}

// Minimum of v over the caller's group of G = 1 << LG lanes (every lane gets it).
template <int LG>
__device__ inline uint32_t group_min(uint32_t v) {
    if constexpr (LG >= 1) v = min(v, lane_xor<1>(v));
    if constexpr (LG >= 2) v = min(v, lane_xor<2>(v));
    if constexpr (LG >= 3) v = min(v, lane_xor<4>(v));
    if constexpr (LG >= 4) v = min(v, lane_xor<8>(v));
    return v;
}

}  // namespace lecb
