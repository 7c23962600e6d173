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

// v plus this lane's bit of the wave mask m (one add with carry-in).
__device__ inline uint32_t plus_lane_bit(uint32_t v, uint64_t m) {
    uint32_t r;
    uint64_t carry_out;
    asm("v_addc_co_u32_e64 %0, %1, %2, 0, %3" : "=v"(r), "=s"(carry_out) : "v"(v), "s"(m));
    (void)carry_out;
    return r;
}

// Exclusive count over the lanes of the caller's group (G = 1 << LG lanes,
// aligned inside a row) of the lanes whose bit of the wave mask `m` is set,
// and the group's total: the group's bits shifted to the bottom of a word,
// then two population counts (a caller's `x + before` folds into the count).
// No lane reads another lane's registers.
template <int LG>
__device__ inline void group_count_mask(uint64_t m, uint32_t& before, uint32_t& total) {
    constexpr uint32_t G = 1u << LG;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t bits = (uint32_t)(m >> (lane & ~(G - 1u)));
    before = (uint32_t)__builtin_popcount(bits & ((1u << (lane & (G - 1u))) - 1u));
    total = (uint32_t)__builtin_popcount(bits & ((1u << G) - 1u));
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

// A DPP move inside rows of 16 lanes (every lane's source is a lane of its
// own row), kept a separate instruction: the compiler's folded form of a DPP
// subtract was measured wrong on gfx950, so no folding is relied on.
template <int CTRL>
__device__ inline uint32_t dpp_row(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Minimum of v over the caller's group of G = 1 << LG lanes (every lane gets
// it), by DPP moves (VALU, no LDS round trip): quad swaps for 2 and 4 lanes,
// a half-row mirror before them for 8, row rotations for 16.
template <int LG>
__device__ inline uint32_t group_min(uint32_t v) {
    if constexpr (LG == 4) {
        v = min(v, dpp_row<0x128>(v));   // row_ror:8
        v = min(v, dpp_row<0x124>(v));   // row_ror:4
        v = min(v, dpp_row<0x122>(v));   // row_ror:2
        v = min(v, dpp_row<0x121>(v));   // row_ror:1
    } else {
        if constexpr (LG == 3) v = min(v, dpp_row<0x141>(v));   // row_half_mirror
        if constexpr (LG >= 1) v = min(v, dpp_row<0xB1>(v));    // quad_perm [1,0,3,2]
        if constexpr (LG >= 2) v = min(v, dpp_row<0x4E>(v));    // quad_perm [2,3,0,1]
    }
    return v;
}

}  // namespace lecb
