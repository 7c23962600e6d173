// Driver for the host runtime built for the CPU alone (codebook.cpp and
// host.cpp with the host compiler and its sanitizers): reads one request per
// line on stdin, answers one line per request on stdout, so that a test can
// compare the answers with the oracle while AddressSanitizer and
// UndefinedBehaviorSanitizer watch every call.  Before the requests it runs
// the argument checks of every entry (null pointers, out-of-range limits,
// corrupt containers) and prints "edges ok".
//
// Requests (all numbers decimal, whitespace separated):
//   build  MAX_LEN MIN_FREQ F[256]        -> rc LEN[256] CODE[256]
//   lens   LEN[256]                       -> rc CODE[256]
//   drift  MAX_LEN TOL_PPM H[256] LEN[256] -> rc refreshed bits_cur bits_opt LEN[256]
//   stats  MAX_LEN H[256] LEN[256]        -> rc n payload_bits optimal_bits uncoded shannon_bits
//   sizes  N CHUNK MAX_LEN                -> num_chunks header_bytes encoded_bound workspace_bytes
//   box    N CHUNK MAX_LEN BYTES_HI BYTES_LO LEN_HI[256] LEN_LO[256]
//                                         -> rc HEADER_HEX, then what reading it back gives
#include <cinttypes>
#include <cstdio>
#include <cstring>
#include <iostream>
#include <sstream>
#include <string>

#include "lecb.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
    if (!ok) {
        std::printf("edge failed: %s\n", what);
        ++failures;
    }
}

void edges() {
    uint64_t hist[256] = {};
    uint8_t len[256] = {};
    lecb_codebook cb{}, out{};
    lecb_stats st{};
    int refreshed = 0;
    uint64_t bc = 0, bo = 0;
    hist[7] = 3;
    hist[9] = 1;
    expect(lecb_build_codebook(nullptr, 16, 0, &cb) == LECB_ERR_INVALID_ARG, "build: null histogram");
    expect(lecb_build_codebook(hist, 16, 0, nullptr) == LECB_ERR_INVALID_ARG, "build: null output");
    expect(lecb_build_codebook(hist, 0, 0, &cb) == LECB_ERR_INVALID_ARG, "build: max_len 0");
    expect(lecb_build_codebook(hist, 17, 0, &cb) == LECB_ERR_INVALID_ARG, "build: max_len 17");
    const uint64_t none[256] = {};
    expect(lecb_build_codebook(none, 16, 0, &cb) == LECB_ERR_NO_SYMBOLS, "build: empty histogram");
    uint64_t all[256];
    for (auto& f : all) f = 1;
    expect(lecb_build_codebook(all, 7, 0, &cb) == LECB_ERR_NO_SYMBOLS, "build: 256 symbols under 7 bits");
    expect(lecb_build_codebook(all, 8, 0, &cb) == LECB_OK, "build: 256 symbols under 8 bits");
    len[0] = 1;
    len[1] = 1;
    len[2] = 1;   // Kraft sum above 1
    expect(lecb_codebook_from_lengths(len, &cb) == LECB_ERR_INVALID_ARG, "lengths: Kraft violated");
    len[2] = 17;
    expect(lecb_codebook_from_lengths(len, &cb) == LECB_ERR_INVALID_ARG, "lengths: length 17");
    expect(lecb_codebook_from_lengths(nullptr, &cb) == LECB_ERR_INVALID_ARG, "lengths: null");
    expect(lecb_build_codebook(hist, 16, 1, &cb) == LECB_OK, "build: fixed codebook");
    expect(lecb_drift_check(nullptr, &cb, 16, 0, &out, &refreshed, &bc, &bo) == LECB_ERR_INVALID_ARG,
           "drift: null histogram");
    expect(lecb_drift_check(hist, &cb, 16, 0, &out, nullptr, &bc, &bo) == LECB_ERR_INVALID_ARG,
           "drift: null flag");
    expect(lecb_drift_check(hist, &cb, 0, 0, &out, &refreshed, &bc, &bo) == LECB_ERR_INVALID_ARG,
           "drift: max_len 0");
    expect(lecb_drift_check(hist, &cb, 16, 0, &cb, &refreshed, nullptr, nullptr) == LECB_OK,
           "drift: in place, no bit counts");
    expect(lecb_stream_stats(hist, nullptr, 16, &st) == LECB_ERR_INVALID_ARG, "stats: null lengths");
    expect(lecb_stream_stats(hist, cb.len, 17, &st) == LECB_ERR_INVALID_ARG, "stats: max_len 17");
    expect(lecb_stream_stats(none, cb.len, 16, &st) == LECB_OK && st.n == 0 && st.shannon_bits == 0.0,
           "stats: empty histogram");
    uint8_t box[LECB_CONTAINER_HEADER_BYTES];
    expect(lecb_container_write_header(nullptr, 1, 4096, 16, cb.len, cb.len, 1, 1) == LECB_ERR_INVALID_ARG,
           "box: null header");
    expect(lecb_container_write_header(box, 1, 4096, 16, cb.len, nullptr, 1, 1) == LECB_ERR_INVALID_ARG,
           "box: null table");
    expect(lecb_container_write_header(box, 1, 4096, 16, cb.len, cb.len, 1, 1) == LECB_OK, "box: write");
    uint64_t n = 0, bh = 0, bl = 0;
    uint32_t chunk = 0, ml = 0;
    uint8_t lh[256], ll[256];
    expect(lecb_container_read_header(box, &n, &chunk, &ml, lh, ll, &bh, nullptr) == LECB_ERR_INVALID_ARG,
           "box: null field");
    box[0] ^= 1;
    expect(lecb_container_read_header(box, &n, &chunk, &ml, lh, ll, &bh, &bl) == LECB_ERR_CORRUPT,
           "box: bad magic");
    box[0] ^= 1;
    box[4] = 2;
    expect(lecb_container_read_header(box, &n, &chunk, &ml, lh, ll, &bh, &bl) == LECB_ERR_CORRUPT,
           "box: bad version");
    for (int s = -20; s <= 2; ++s) expect(lecb_status_str(s) != nullptr, "status text");
    expect(lecb_num_chunks(UINT64_MAX, 256) == (UINT64_MAX >> 8) + 1, "chunks of 2^64 - 1 symbols");
    expect(lecb_num_chunks(100, 300) == 0 && lecb_header_bytes(100, 128) == 0, "sizes: bad chunk");
    expect(lecb_encoded_bound(1ull << 60, 4096, 16) == 0, "bound: n at 2^60");
    expect(lecb_encoded_bound((1ull << 60) - 1, 256, 16) > (1ull << 60), "bound: largest n");
    expect(lecb_workspace_bytes(UINT64_MAX, 65536) > 0, "workspace: largest n");
    expect(lecb_abi_version() == LECB_ABI_VERSION, "abi version");
    expect(lecb_device_codebook_bytes() % 16 == 0, "device codebook size");
}

template <typename T>
bool read_n(std::istringstream& in, T* v, int n) {
    for (int i = 0; i < n; ++i) {
        uint64_t x;
        if (!(in >> x)) return false;
        v[i] = (T)x;
    }
    return true;
}

void print_lens(const uint8_t* len) {
    for (int s = 0; s < 256; ++s) std::printf(" %u", len[s]);
}

void print_codes(const lecb_codebook& cb) {
    for (int s = 0; s < 256; ++s) std::printf(" %u", cb.code[s]);
}

}  // namespace

int main() {
    edges();
    std::printf(failures ? "edges failed\n" : "edges ok\n");
    std::string line;
    while (std::getline(std::cin, line)) {
        std::istringstream in(line);
        std::string op;
        if (!(in >> op)) continue;
        if (op == "build") {
            uint32_t ml, mf;
            uint64_t f[256];
            in >> ml >> mf;
            if (!read_n(in, f, 256)) return 2;
            lecb_codebook cb{};
            const int rc = lecb_build_codebook(f, ml, mf, &cb);
            std::printf("%d", rc);
            print_lens(cb.len);
            print_codes(cb);
        } else if (op == "lens") {
            uint8_t len[256];
            if (!read_n(in, len, 256)) return 2;
            lecb_codebook cb{};
            std::printf("%d", lecb_codebook_from_lengths(len, &cb));
            print_codes(cb);
        } else if (op == "drift") {
            uint32_t ml, tol;
            uint64_t h[256];
            lecb_codebook cur{}, out{};
            in >> ml >> tol;
            if (!read_n(in, h, 256) || !read_n(in, cur.len, 256)) return 2;
            int refreshed = -1;
            uint64_t bc = 0, bo = 0;
            const int rc = lecb_drift_check(h, &cur, ml, tol, &out, &refreshed, &bc, &bo);
            std::printf("%d %d %" PRIu64 " %" PRIu64, rc, refreshed, bc, bo);
            print_lens(out.len);
        } else if (op == "stats") {
            uint32_t ml;
            uint64_t h[256];
            uint8_t len[256];
            in >> ml;
            if (!read_n(in, h, 256) || !read_n(in, len, 256)) return 2;
            lecb_stats st{};
            const int rc = lecb_stream_stats(h, len, ml, &st);
            std::printf("%d %" PRIu64 " %" PRIu64 " %" PRIu64 " %" PRIu64 " %.17g", rc, st.n, st.payload_bits,
                        st.optimal_bits, st.uncoded, st.shannon_bits);
        } else if (op == "sizes") {
            uint64_t n;
            uint32_t chunk, ml;
            in >> n >> chunk >> ml;
            std::printf("%" PRIu64 " %" PRIu64 " %" PRIu64 " %" PRIu64, lecb_num_chunks(n, chunk),
                        lecb_header_bytes(n, chunk), lecb_encoded_bound(n, chunk, ml),
                        lecb_workspace_bytes(n, chunk));
        } else if (op == "box") {
            uint64_t n, bh, bl;
            uint32_t chunk, ml;
            uint8_t lh[256], ll[256];
            in >> n >> chunk >> ml >> bh >> bl;
            if (!read_n(in, lh, 256) || !read_n(in, ll, 256)) return 2;
            uint8_t box[LECB_CONTAINER_HEADER_BYTES];
            std::printf("%d ", lecb_container_write_header(box, n, chunk, ml, lh, ll, bh, bl));
            for (uint8_t b : box) std::printf("%02x", b);
            uint64_t n2 = 0, bh2 = 0, bl2 = 0;
            uint32_t c2 = 0, ml2 = 0;
            uint8_t lh2[256], ll2[256];
            const int rc = lecb_container_read_header(box, &n2, &c2, &ml2, lh2, ll2, &bh2, &bl2);
            std::printf(" %d %" PRIu64 " %u %u %" PRIu64 " %" PRIu64, rc, n2, c2, ml2, bh2, bl2);
            print_lens(lh2);
            print_lens(ll2);
        } else {
            return 2;
        }
        std::printf("\n");
    }
    return failures ? 1 : 0;
}
