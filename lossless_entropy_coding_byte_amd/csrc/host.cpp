// Host-only entries of the C ABI that touch no device: version, status text,
// stream and workspace sizes.  Plain C++ (no HIP header), so that this file
// and codebook.cpp also build with the host compiler alone, as the sanitized
// CPU build of the host runtime does.
#include <cstdint>

#include "lecb.h"
#include "lecb_internal.hpp"

using namespace lecb;

extern "C" {

uint32_t lecb_abi_version(void) { return LECB_ABI_VERSION; }

const char* lecb_status_str(int status) {
    switch (status) {
        case LECB_OK: return "ok";
        case LECB_ERR_INVALID_ARG: return "invalid argument";
        case LECB_ERR_CAPACITY: return "output capacity too small";
        case LECB_ERR_TOO_LARGE: return "payload needs 2^32 words or more";
        case LECB_ERR_NO_SYMBOLS: return "no codebook possible for this histogram";
        case LECB_ERR_HIP: return "HIP runtime error";
        case LECB_ERR_WORKSPACE: return "workspace too small";
        case LECB_ERR_SCRATCH: return "input too large for the static scratch of the no-allocation encode";
        case LECB_ERR_UNCODED_SYMBOL: return "input holds a byte with no code word";
        case LECB_ERR_CORRUPT: return "corrupt stream";
        default: return "unknown status";
    }
}

uint64_t lecb_num_chunks(uint64_t n, uint32_t chunk) { return num_chunks_of(n, chunk); }

uint64_t lecb_header_bytes(uint64_t n, uint32_t chunk) { return header_bytes_of(n, chunk); }

uint64_t lecb_encoded_bound(uint64_t n, uint32_t chunk, uint32_t max_len) {
    // below 2^60 symbols every term stays far from 2^64
    if (!valid_chunk(chunk) || max_len < 1 || max_len > 16 || n >= (1ull << 60)) return 0;
    const uint64_t nc = num_chunks_of(n, chunk);
    if (!nc) return 0;
    // a lane of m symbols takes at most ceil(m * max_len / 32) words; every
    // chunk but the last has G lanes of chunk / G symbols
    const uint64_t G = lanes_per_chunk(chunk);
    uint64_t words = (nc - 1) * G * (((uint64_t)chunk / G * max_len + 31) / 32);
    const uint64_t last = n - (nc - 1) * chunk;   // symbols of the last chunk
    const uint64_t full = last / 16, rest = last % 16;
    for (uint64_t j = 0; j < G; ++j) {
        const uint64_t whole = full > j ? (full - j + G - 1) / G : 0;
        const uint64_t m = whole * 16 + ((full % G) == j && rest ? rest : 0);
        words += (m * max_len + 31) / 32;
    }
    return align16(header_bytes_of(n, chunk) + 4 * words);
}

uint64_t lecb_workspace_bytes(uint64_t n, uint32_t chunk) {
    return valid_chunk(chunk) ? ws_bytes_of(n, chunk) : 0;
}

uint64_t lecb_device_codebook_bytes(void) { return sizeof(DeviceCodebook); }

}  // extern "C"
