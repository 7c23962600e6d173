// Host-side codebook construction: frequency clamp, length-limited optimal
// code lengths, canonical code words, container header.
//
// Basis: "Single-Stage Huffman Encoder for ML Compression", Methodology
// steps 2-3 (one codebook built once from the combined warm-up statistics)
// and "Lossless Compression for LLM Tensor Incremental Snapshots", Technical
// framework step 3 / Key design item 2 (an efficient Huffman-tree build).
//
// Length limiting uses package-merge (Larmore & Hirschberg 1990) in its
// O(L*m) form: for each denomination level we keep only the merged order of
// coins and packages; the selected prefix of a level always consists of the
// cheapest `a` coins and the first `p` packages, and those packages are the
// first 2p items of the level below.  A coin's code length is the number of
// levels whose selected prefix contains it.  Tie rule (fixed so the result is
// unique): coins are ordered by (frequency, byte value); at equal weight a
// coin is placed before a package.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "lecb.h"
#include "lecb_internal.hpp"

namespace lecb {

int build_lengths(const uint64_t freq_in[256], uint32_t max_len, uint32_t min_freq,
                  uint8_t len_out[256]) {
    if (!freq_in || !len_out || max_len < 1 || max_len > 16) return LECB_ERR_INVALID_ARG;
    uint64_t freq[256];
    for (int s = 0; s < 256; ++s) freq[s] = std::max<uint64_t>(freq_in[s], min_freq);
    std::memset(len_out, 0, 256);

    int order[256];
    int m = 0;
    for (int s = 0; s < 256; ++s)
        if (freq[s] > 0) order[m++] = s;
    if (m == 0) return LECB_ERR_NO_SYMBOLS;
    if (m == 1) {
        len_out[order[0]] = 1;
        return LECB_OK;
    }
    if ((uint64_t)m > (1ull << max_len)) return LECB_ERR_NO_SYMBOLS;
    std::stable_sort(order, order + m, [&](int a, int b) { return freq[a] < freq[b]; });

    // is_pkg[k][i]: item i of level k's merged order is a package (else a
    // coin).  A level holds m coins and at most m - 1 packages.
    const int L = (int)max_len;
    static thread_local uint8_t is_pkg[16][512];
    static thread_local uint64_t wbuf[2][512];
    int len_at[16];
    uint64_t* cur_w = wbuf[0];
    uint64_t* next_w = wbuf[1];
    uint64_t coin_w[256];
    for (int i = 0; i < m; ++i) coin_w[i] = freq[order[i]];
    int cur_n = m;
    for (int i = 0; i < m; ++i) {
        cur_w[i] = coin_w[i];
        is_pkg[0][i] = 0;
    }
    len_at[0] = m;
    for (int k = 1; k < L; ++k) {
        const int np = cur_n / 2;
        int ic = 0, ip = 0, o = 0;
        // package weights are formed on the fly from consecutive pairs of cur_w
        while (ic < m || ip < np) {
            const uint64_t pw = ip < np ? cur_w[2 * ip] + cur_w[2 * ip + 1] : 0;
            const bool take_coin = ip == np || (ic < m && coin_w[ic] <= pw);
            if (take_coin) {
                next_w[o] = coin_w[ic++];
                is_pkg[k][o++] = 0;
            } else {
                next_w[o] = pw;
                is_pkg[k][o++] = 1;
                ++ip;
            }
        }
        len_at[k] = o;
        cur_n = o;
        std::swap(cur_w, next_w);
    }

    // Walk down from the top level: take the first `take` items of each level.
    size_t take = 2 * (size_t)m - 2;
    int coins_at[16] = {0};
    for (int k = L - 1; k >= 0; --k) {
        if (take > (size_t)len_at[k]) return LECB_ERR_NO_SYMBOLS;  // cannot happen when m <= 2^L
        size_t a = 0, p = 0;
        for (size_t i = 0; i < take; ++i) (is_pkg[k][i] ? p : a) += 1;
        coins_at[k] = (int)a;
        take = 2 * p;
    }
    for (int i = 0; i < m; ++i) {
        int l = 0;
        for (int k = 0; k < L; ++k) l += i < coins_at[k];
        len_out[order[i]] = (uint8_t)l;
    }
    return LECB_OK;
}

int canonical_from_lengths(const uint8_t len[256], lecb_codebook* out) {
    if (!len || !out) return LECB_ERR_INVALID_ARG;
    int count[17] = {0};
    uint32_t maxl = 0, coded = 0;
    for (int s = 0; s < 256; ++s) {
        if (len[s] > 16) return LECB_ERR_INVALID_ARG;
        if (len[s]) {
            ++count[len[s]];
            ++coded;
            maxl = std::max<uint32_t>(maxl, len[s]);
        }
    }
    // Kraft: sum 2^(16-l) <= 2^16
    uint64_t kraft = 0;
    for (int l = 1; l <= 16; ++l) kraft += (uint64_t)count[l] << (16 - l);
    if (kraft > (1ull << 16)) return LECB_ERR_INVALID_ARG;
    // first code of each length: codes of length l follow those of length l-1
    uint32_t next[17] = {0};
    uint32_t code = 0;
    for (int l = 1; l <= 16; ++l) {
        code = (code + count[l - 1]) << 1;
        next[l] = code;
    }
    std::memset(out, 0, sizeof(*out));
    for (int s = 0; s < 256; ++s) {  // ascending byte value within each length
        const int l = len[s];
        out->len[s] = (uint8_t)l;
        if (l) out->code[s] = (uint16_t)next[l]++;
    }
    out->num_coded = coded;
    out->max_len = maxl ? maxl : 1;
    return LECB_OK;
}

}  // namespace lecb

extern "C" {

int lecb_build_codebook(const uint64_t hist[256], uint32_t max_len, uint32_t min_freq,
                        lecb_codebook* out) {
    if (!hist || !out) return LECB_ERR_INVALID_ARG;
    uint8_t len[256];
    const int rc = lecb::build_lengths(hist, max_len, min_freq, len);
    if (rc != LECB_OK) return rc;
    const int rc2 = lecb::canonical_from_lengths(len, out);
    if (rc2 != LECB_OK) return rc2;
    out->max_len = max_len;
    return LECB_OK;
}

int lecb_codebook_from_lengths(const uint8_t len[256], lecb_codebook* out) {
    return lecb::canonical_from_lengths(len, out);
}

// Refresh rule for a drifting stream ("Single-Stage Huffman Encoder for ML
// Compression", Limitations and future work: distribution drift; the page
// leaves the rule open).  The batch keeps the current codebook unless its
// payload bits under it exceed, by more than tol_ppm, those of the best fixed
// codebook for the batch: package-merge on the batch histogram clamped to
// frequency >= 1 (built like every fixed codebook).  Integer decision:
// bits_cur * 10^6 > bits_opt * (10^6 + tol_ppm).
int lecb_drift_check(const uint64_t hist[256], const lecb_codebook* cur, uint32_t max_len,
                     uint32_t tol_ppm, lecb_codebook* out, int* refreshed, uint64_t* bits_cur,
                     uint64_t* bits_opt) {
    if (!hist || !cur || !out || !refreshed || max_len < 1 || max_len > 16) return LECB_ERR_INVALID_ARG;
    lecb_codebook best;
    const int rc = lecb_build_codebook(hist, max_len, 1, &best);
    if (rc != LECB_OK) return rc;
    unsigned __int128 bc = 0, bo = 0;
    bool codable = true;
    for (int s = 0; s < 256; ++s) {
        if (hist[s] && !cur->len[s]) codable = false;
        bc += (unsigned __int128)hist[s] * cur->len[s];
        bo += (unsigned __int128)hist[s] * best.len[s];
    }
    const bool refresh =
        !codable || bc * 1000000u > bo * (unsigned __int128)(1000000ull + tol_ppm);
    if (refresh) {
        *out = best;
    } else if (out != cur) {
        *out = *cur;
    }
    *refreshed = refresh ? 1 : 0;
    if (bits_cur) *bits_cur = codable ? (uint64_t)bc : UINT64_MAX;
    if (bits_opt) *bits_opt = (uint64_t)bo;
    return LECB_OK;
}

int lecb_stream_stats(const uint64_t hist[256], const uint8_t len[256], uint32_t max_len,
                      lecb_stats* out) {
    if (!hist || !len || !out || max_len < 1 || max_len > 16) return LECB_ERR_INVALID_ARG;
    std::memset(out, 0, sizeof(*out));
    for (int s = 0; s < 256; ++s) {
        out->n += hist[s];
        out->payload_bits += hist[s] * len[s];
        if (!len[s]) out->uncoded += hist[s];
    }
    if (out->n) {
        const double n = (double)out->n;
        double h = 0.0;
        for (int s = 0; s < 256; ++s) {
            if (hist[s]) {
                const double p = (double)hist[s] / n;
                h -= p * std::log2(p);
            }
        }
        out->shannon_bits = n * h;
        uint8_t opt[256];
        const int rc = lecb::build_lengths(hist, max_len, 0, opt);
        if (rc == LECB_OK)
            for (int s = 0; s < 256; ++s) out->optimal_bits += hist[s] * opt[s];
    }
    return LECB_OK;
}

static void put_u16(uint8_t* p, uint16_t v) { std::memcpy(p, &v, 2); }
static void put_u32(uint8_t* p, uint32_t v) { std::memcpy(p, &v, 4); }
static void put_u64(uint8_t* p, uint64_t v) { std::memcpy(p, &v, 8); }

int lecb_container_write_header(uint8_t out[LECB_CONTAINER_HEADER_BYTES], uint64_t n,
                                uint32_t chunk, uint32_t max_len, const uint8_t len_hi[256],
                                const uint8_t len_lo[256], uint64_t bytes_hi,
                                uint64_t bytes_lo) {
    if (!out || !len_hi || !len_lo) return LECB_ERR_INVALID_ARG;
    std::memset(out, 0, LECB_CONTAINER_HEADER_BYTES);
    std::memcpy(out, "LECB", 4);
    put_u16(out + 4, 1);
    put_u16(out + 6, 1);
    put_u64(out + 8, n);
    put_u32(out + 16, chunk);
    put_u32(out + 20, max_len);
    std::memcpy(out + 24, len_hi, 256);
    std::memcpy(out + 280, len_lo, 256);
    put_u64(out + 536, bytes_hi);
    put_u64(out + 544, bytes_lo);
    return LECB_OK;
}

int lecb_container_read_header(const uint8_t in[LECB_CONTAINER_HEADER_BYTES], uint64_t* n,
                               uint32_t* chunk, uint32_t* max_len, uint8_t len_hi[256],
                               uint8_t len_lo[256], uint64_t* bytes_hi, uint64_t* bytes_lo) {
    if (!in || !n || !chunk || !max_len || !len_hi || !len_lo || !bytes_hi || !bytes_lo)
        return LECB_ERR_INVALID_ARG;
    uint16_t ver, kind;
    std::memcpy(&ver, in + 4, 2);
    std::memcpy(&kind, in + 6, 2);
    if (std::memcmp(in, "LECB", 4) != 0 || ver != 1 || kind != 1) return LECB_ERR_CORRUPT;
    std::memcpy(n, in + 8, 8);
    std::memcpy(chunk, in + 16, 4);
    std::memcpy(max_len, in + 20, 4);
    std::memcpy(len_hi, in + 24, 256);
    std::memcpy(len_lo, in + 280, 256);
    std::memcpy(bytes_hi, in + 536, 8);
    std::memcpy(bytes_lo, in + 544, 8);
    return LECB_OK;
}

}  // extern "C"
