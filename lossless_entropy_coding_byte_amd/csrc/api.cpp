// C ABI: argument checks, sizes, workspace, launches.  No device allocation,
// no implicit synchronisation (lecb_encode_bf16_pertensor aside).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "lecb.h"
#include "lecb_internal.hpp"

using namespace lecb;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Histograms come back through a pinned buffer (one per host thread, 8 KiB,
// allocated on first use and kept): a direct DMA, no staging copy.  Waits for
// `stream`.
int read_back_hist(const uint64_t* d_hist, int count, void* stream, const uint64_t** host) {
    thread_local uint64_t* h = nullptr;
    if (count > 1024) return LECB_ERR_INVALID_ARG;
    if (!h && hipHostMalloc(reinterpret_cast<void**>(&h), 1024 * sizeof(uint64_t), hipHostMallocDefault) != hipSuccess) {
        h = nullptr;
        return LECB_ERR_HIP;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(h, d_hist, count * sizeof(uint64_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return LECB_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return LECB_ERR_HIP;
    *host = h;
    return LECB_OK;
}

int build_args(const lecb_codebook* cb, CodebookArgs* a) {
    lecb_codebook canon;
    const int rc = canonical_from_lengths(cb->len, &canon);
    if (rc != LECB_OK) return rc;
    std::memset(a, 0, sizeof(*a));
    for (int s = 0; s < 256; ++s) {
        a->enc[s] = canon.len[s] ? ((uint32_t)canon.code[s] << 5) | canon.len[s] : 0u;
        if (canon.len[s]) ++a->count[canon.len[s]];
    }
    uint32_t code = 0, idx = 0;
    for (int l = 1; l <= 16; ++l) {
        code = (code + a->count[l - 1]) << 1;
        a->first[l] = code;
        a->base[l] = idx;
        idx += a->count[l];
    }
    uint32_t fill[17];
    std::memcpy(fill, a->base, sizeof(fill));
    for (int s = 0; s < 256; ++s)
        if (canon.len[s]) a->sorted[fill[canon.len[s]]++] = (uint8_t)s;
    a->max_len = 0;
    for (int s = 0; s < 256; ++s) a->max_len = std::max<uint32_t>(a->max_len, canon.len[s]);
    a->num_coded = canon.num_coded;
    return LECB_OK;
}

int encode_common(const void* d_in, int mode, uint64_t n, const void* d_blob, uint32_t chunk,
                  uint8_t* d_out, uint64_t out_capacity, lecb_result* d_res, void* d_ws,
                  uint64_t ws_bytes, void* stream, const void* d_blob2 = nullptr,
                  uint8_t* d_out2 = nullptr, uint64_t out_capacity2 = 0, const void* d_in2 = nullptr) {
    const bool pair = two_stream_mode(mode);
    if (mode == ENC_PAIR_XOR && n && (!d_in2 || !aligned16(d_in2))) return LECB_ERR_INVALID_ARG;
    if (!valid_chunk(chunk) || !d_res || !d_blob || !aligned16(d_blob)) return LECB_ERR_INVALID_ARG;
    if (pair && (!d_blob2 || !aligned16(d_blob2))) return LECB_ERR_INVALID_ARG;
    if (n == 0) {
        int rc = launch_result(d_res, 0, 0, LECB_OK, stream);
        return (rc || !pair) ? rc : launch_result(d_res + 1, 0, 0, LECB_OK, stream);
    }
    if (!d_in || !d_out || !d_ws || !aligned16(d_in) || !aligned16(d_out) || !aligned16(d_ws))
        return LECB_ERR_INVALID_ARG;
    if (pair && (!d_out2 || !aligned16(d_out2))) return LECB_ERR_INVALID_ARG;
    const uint64_t nc = num_chunks_of(n, chunk);
    if (ws_bytes < ws_bytes_of(n, chunk)) return LECB_ERR_WORKSPACE;
    if (out_capacity < header_bytes_of(n, chunk)) return LECB_ERR_CAPACITY;
    if (pair && out_capacity2 < header_bytes_of(n, chunk)) return LECB_ERR_CAPACITY;
    EncodeLaunch L{};
    L.in = d_in;
    L.in2 = d_in2;
    L.mode = mode;
    L.n = n;
    L.chunk = chunk;
    L.nc = nc;
    L.st[0].cb = reinterpret_cast<const DeviceCodebook*>(d_blob);
    L.st[0].out = d_out;
    L.st[0].capacity = out_capacity;
    L.st[0].res = d_res;
    L.st[0].ws = reinterpret_cast<WsHeader*>(d_ws);
    if (pair) {
        L.st[1].cb = reinterpret_cast<const DeviceCodebook*>(d_blob2);
        L.st[1].out = d_out2;
        L.st[1].capacity = out_capacity2;
        L.st[1].res = d_res + 1;
        L.st[1].ws = reinterpret_cast<WsHeader*>(static_cast<uint8_t*>(d_ws) + ws_stream_bytes(nc));
    }
    return launch_encode(L, stream);
}

// Decode ns streams of the same n and chunk in one launch: into their own
// byte outputs (DEC_OUT_PLANES), or restored into the elements `merged`.
int decode_common(int ns, int kind, const uint8_t* const* d_stream, const uint64_t* stream_bytes,
                  const void* const* d_blob, uint32_t chunk, uint64_t n, uint8_t* const* d_out,
                  uint8_t* merged, const uint8_t* w0, lecb_result* d_res, void* d_ws, uint64_t ws_bytes,
                  void* stream, const lecb_result* d_sizes = nullptr) {
    if (!valid_chunk(chunk) || !d_res) return LECB_ERR_INVALID_ARG;
    for (int k = 0; k < ns; ++k)
        if (!d_blob[k] || !aligned16(d_blob[k])) return LECB_ERR_INVALID_ARG;
    if (n == 0) {
        for (int k = 0; k < ns; ++k) {
            // (with device-side sizes the encoder of 0 symbols wrote an empty result)
            const int rc = launch_result(d_res + k, 0, 0,
                                         d_sizes || stream_bytes[k] == 0 ? LECB_OK : LECB_ERR_CORRUPT,
                                         stream);
            if (rc) return rc;
        }
        return LECB_OK;
    }
    if (!d_ws || !aligned16(d_ws)) return LECB_ERR_INVALID_ARG;
    if (kind != DEC_OUT_PLANES && (!merged || !aligned16(merged))) return LECB_ERR_INVALID_ARG;
    if (kind == DEC_OUT_U16_XOR && (!w0 || !aligned16(w0))) return LECB_ERR_INVALID_ARG;
    const uint64_t hb = header_bytes_of(n, chunk);
    for (int k = 0; k < ns; ++k) {
        if (!d_stream[k] || !aligned16(d_stream[k])) return LECB_ERR_INVALID_ARG;
        if (kind == DEC_OUT_PLANES && (!d_out[k] || !aligned16(d_out[k]))) return LECB_ERR_INVALID_ARG;
        if (!d_sizes && (stream_bytes[k] < hb + 4 || (stream_bytes[k] - hb) % 4)) return LECB_ERR_CORRUPT;
    }
    if (ws_bytes < ws_bytes_of(n, chunk)) return LECB_ERR_WORKSPACE;
    const uint64_t nc = num_chunks_of(n, chunk);
    if (d_sizes && !aligned16(d_sizes)) return LECB_ERR_INVALID_ARG;
    DecodeLaunch L{};
    L.nstreams = ns;
    L.out_kind = kind;
    L.dev_sizes = d_sizes;
    L.merged = merged;
    L.w0 = w0;
    for (int k = 0; k < ns; ++k) {
        L.stream_base[k] = d_stream[k];
        L.stream_bytes[k] = d_sizes ? 0 : stream_bytes[k];
        L.cb[k] = reinterpret_cast<const DeviceCodebook*>(d_blob[k]);
        L.out[k] = kind == DEC_OUT_PLANES ? d_out[k] : nullptr;
        L.res[k] = d_res + k;
        L.ws[k] = reinterpret_cast<WsHeader*>(static_cast<uint8_t*>(d_ws) + ws_header_offset(k, nc));
    }
    L.chunk = chunk;
    L.n = n;
    L.nc = nc;
    return launch_decode(L, stream);
}

}  // namespace

// Per-tensor two-plane encode of d_in (d_in2 == nullptr) or of d_in ^ d_in2.
static int pertensor_common(const uint16_t* d_in, const uint16_t* d_in2, uint64_t n, uint32_t chunk,
                               uint32_t max_len, uint64_t* d_hist, void* d_blob_hi,
                               void* d_blob_lo, lecb_codebook* cb_hi, lecb_codebook* cb_lo,
                               uint8_t* d_out_hi, uint64_t cap_hi, uint8_t* d_out_lo,
                               uint64_t cap_lo, lecb_result* d_res2, void* d_ws,
                               uint64_t ws_bytes, void* stream) {
    if (!valid_chunk(chunk) || max_len < 1 || max_len > 16 || !d_hist || !aligned16(d_hist) ||
        !cb_hi || !cb_lo || !d_res2)
        return LECB_ERR_INVALID_ARG;
    if (n == 0) {
        std::memset(cb_hi, 0, sizeof(*cb_hi));
        std::memset(cb_lo, 0, sizeof(*cb_lo));
        int rc = launch_result(d_res2, 0, 0, LECB_OK, stream);
        return rc ? rc : launch_result(d_res2 + 1, 0, 0, LECB_OK, stream);
    }
    int rc = d_in2 ? lecb_histogram_bf16_delta(d_in, d_in2, n, d_hist, d_hist + 256, 0, stream)
                   : lecb_histogram_bf16(d_in, n, d_hist, d_hist + 256, 0, stream);
    if (rc) return rc;
    const uint64_t* h = nullptr;
    rc = read_back_hist(d_hist, 512, stream, &h);
    if (rc) return rc;
    // d_hist[0:256] = high plane, d_hist[256:512] = low plane
    rc = lecb_build_codebook(h, max_len, 0, cb_hi);
    if (!rc) rc = lecb_build_codebook(h + 256, max_len, 0, cb_lo);
    if (!rc) rc = lecb_codebook_upload(cb_hi, d_blob_hi, stream);
    if (!rc) rc = lecb_codebook_upload(cb_lo, d_blob_lo, stream);
    if (!rc)
        rc = d_in2 ? lecb_encode_bf16_delta(d_in, d_in2, n, d_blob_hi, d_blob_lo, chunk, d_out_hi,
                                            cap_hi, d_out_lo, cap_lo, d_res2, d_ws, ws_bytes, stream)
                   : lecb_encode_bf16(d_in, n, d_blob_hi, d_blob_lo, chunk, d_out_hi, cap_hi, d_out_lo,
                                      cap_lo, d_res2, d_ws, ws_bytes, stream);
    return rc;
}

extern "C" {

int lecb_workspace_init(void* d_ws, uint64_t ws_bytes, void* stream) {
    if (!d_ws || !aligned16(d_ws) || ws_bytes < sizeof(WsHeader)) return LECB_ERR_INVALID_ARG;
    return launch_fill_zero(d_ws, ws_bytes, stream);
}

int lecb_codebook_upload(const lecb_codebook* cb, void* d_blob, void* stream) {
    if (!cb || !d_blob || !aligned16(d_blob)) return LECB_ERR_INVALID_ARG;
    CodebookArgs args;
    const int rc = build_args(cb, &args);
    if (rc != LECB_OK) return rc;
    return launch_codebook_upload(args, reinterpret_cast<DeviceCodebook*>(d_blob), stream);
}

int lecb_histogram(const uint8_t* d_in, uint64_t n, uint64_t* d_hist, int accumulate,
                   void* stream) {
    if (!d_hist || !aligned16(d_hist) || (n && (!d_in || !aligned16(d_in))))
        return LECB_ERR_INVALID_ARG;
    return launch_histogram_u8(d_in, n, d_hist, accumulate, stream);
}

int lecb_histogram_bf16(const uint16_t* d_in, uint64_t n, uint64_t* d_hist_hi,
                        uint64_t* d_hist_lo, int accumulate, void* stream) {
    if (!d_hist_hi || !d_hist_lo || !aligned16(d_hist_hi) || !aligned16(d_hist_lo) ||
        (n && (!d_in || !aligned16(d_in))))
        return LECB_ERR_INVALID_ARG;
    return launch_histogram_u16(d_in, nullptr, n, d_hist_hi, d_hist_lo, accumulate, stream);
}

int lecb_split_bf16(const uint16_t* d_in, uint64_t n, uint8_t* d_hi, uint8_t* d_lo,
                    void* stream) {
    if (n && (!d_in || !d_hi || !d_lo || !aligned16(d_in) || !aligned16(d_hi) || !aligned16(d_lo)))
        return LECB_ERR_INVALID_ARG;
    return launch_split(d_in, n, d_hi, d_lo, stream);
}

int lecb_merge_bf16(const uint8_t* d_hi, const uint8_t* d_lo, uint64_t n, uint16_t* d_out,
                    void* stream) {
    if (n && (!d_out || !d_hi || !d_lo || !aligned16(d_out) || !aligned16(d_hi) || !aligned16(d_lo)))
        return LECB_ERR_INVALID_ARG;
    return launch_merge(d_hi, d_lo, nullptr, n, d_out, stream);
}

int lecb_encode(const uint8_t* d_in, uint64_t n, const void* d_blob, uint32_t chunk,
                uint8_t* d_out, uint64_t out_capacity, lecb_result* d_res, void* d_ws,
                uint64_t ws_bytes, void* stream) {
    return encode_common(d_in, ENC_BYTES, n, d_blob, chunk, d_out, out_capacity, d_res, d_ws, ws_bytes,
                         stream);
}

int lecb_encode_plane(const uint16_t* d_in, uint64_t n, int plane, const void* d_blob,
                      uint32_t chunk, uint8_t* d_out, uint64_t out_capacity,
                      lecb_result* d_res, void* d_ws, uint64_t ws_bytes, void* stream) {
    if (plane != 0 && plane != 1) return LECB_ERR_INVALID_ARG;
    return encode_common(d_in, plane ? ENC_PLANE_HI : ENC_PLANE_LO, n, d_blob, chunk, d_out,
                         out_capacity, d_res, d_ws,
                         ws_bytes, stream);
}

int lecb_encode_bf16(const uint16_t* d_in, uint64_t n, const void* d_blob_hi,
                     const void* d_blob_lo, uint32_t chunk, uint8_t* d_out_hi, uint64_t cap_hi,
                     uint8_t* d_out_lo, uint64_t cap_lo, lecb_result* d_res2, void* d_ws,
                     uint64_t ws_bytes, void* stream) {
    return encode_common(d_in, ENC_PAIR, n, d_blob_hi, chunk, d_out_hi, cap_hi, d_res2, d_ws,
                         ws_bytes, stream, d_blob_lo, d_out_lo, cap_lo);
}

int lecb_decode(const uint8_t* d_stream, uint64_t stream_bytes, const void* d_blob,
                uint32_t chunk, uint64_t n, uint8_t* d_out, lecb_result* d_res, void* d_ws,
                uint64_t ws_bytes, void* stream) {
    const uint8_t* st[1] = {d_stream};
    const uint64_t sb[1] = {stream_bytes};
    const void* bl[1] = {d_blob};
    uint8_t* out[1] = {d_out};
    return decode_common(1, DEC_OUT_PLANES, st, sb, bl, chunk, n, out, nullptr, nullptr, d_res, d_ws, ws_bytes,
                         stream);
}

int lecb_decode_from_result(const uint8_t* d_stream, const lecb_result* d_enc_res,
                            const void* d_blob, uint32_t chunk, uint64_t n, uint8_t* d_out,
                            lecb_result* d_res, void* d_ws, uint64_t ws_bytes, void* stream) {
    if (!d_enc_res) return LECB_ERR_INVALID_ARG;
    const uint8_t* st[1] = {d_stream};
    const uint64_t sb[1] = {0};
    const void* bl[1] = {d_blob};
    uint8_t* out[1] = {d_out};
    return decode_common(1, DEC_OUT_PLANES, st, sb, bl, chunk, n, out, nullptr, nullptr, d_res, d_ws, ws_bytes,
                         stream, d_enc_res);
}

int lecb_decode_bf16_from_results(const uint8_t* d_hi, const uint8_t* d_lo,
                                  const lecb_result* d_enc_res2, const void* d_blob_hi,
                                  const void* d_blob_lo, uint32_t chunk, uint64_t n,
                                  uint16_t* d_out, lecb_result* d_res2,
                                  void* d_ws, uint64_t ws_bytes, void* stream) {
    if (!d_res2 || !d_enc_res2) return LECB_ERR_INVALID_ARG;
    const uint8_t* st[2] = {d_hi, d_lo};
    const uint64_t sb[2] = {0, 0};
    const void* bl[2] = {d_blob_hi, d_blob_lo};
    return decode_common(2, DEC_OUT_U16, st, sb, bl, chunk, n, nullptr, reinterpret_cast<uint8_t*>(d_out), nullptr,
                         d_res2, d_ws, ws_bytes, stream, d_enc_res2);
}

int lecb_decode_bf16_delta_from_results(const uint8_t* d_hi, const uint8_t* d_lo,
                                        const lecb_result* d_enc_res2, const void* d_blob_hi,
                                        const void* d_blob_lo, uint32_t chunk, uint64_t n,
                                        const uint16_t* d_w0, uint16_t* d_w1,
                                        lecb_result* d_res2, void* d_ws, uint64_t ws_bytes,
                                        void* stream) {
    if (!d_res2 || !d_enc_res2) return LECB_ERR_INVALID_ARG;
    if (n && d_w0 == d_w1) return LECB_ERR_INVALID_ARG;
    const uint8_t* st[2] = {d_hi, d_lo};
    const uint64_t sb[2] = {0, 0};
    const void* bl[2] = {d_blob_hi, d_blob_lo};
    return decode_common(2, DEC_OUT_U16_XOR, st, sb, bl, chunk, n, nullptr, reinterpret_cast<uint8_t*>(d_w1),
                         reinterpret_cast<const uint8_t*>(d_w0), d_res2, d_ws, ws_bytes, stream, d_enc_res2);
}

int lecb_decode_bf16_delta(const uint8_t* d_hi, uint64_t hi_bytes, const uint8_t* d_lo,
                           uint64_t lo_bytes, const void* d_blob_hi, const void* d_blob_lo,
                           uint32_t chunk, uint64_t n, const uint16_t* d_w0, uint16_t* d_w1,
                           lecb_result* d_res2, void* d_ws, uint64_t ws_bytes,
                           void* stream) {
    if (!d_res2) return LECB_ERR_INVALID_ARG;
    if (n && d_w0 == d_w1) return LECB_ERR_INVALID_ARG;
    const uint8_t* st[2] = {d_hi, d_lo};
    const uint64_t sb[2] = {hi_bytes, lo_bytes};
    const void* bl[2] = {d_blob_hi, d_blob_lo};
    return decode_common(2, DEC_OUT_U16_XOR, st, sb, bl, chunk, n, nullptr, reinterpret_cast<uint8_t*>(d_w1),
                         reinterpret_cast<const uint8_t*>(d_w0), d_res2, d_ws, ws_bytes, stream);
}

int lecb_decode_bf16_planes(const uint8_t* d_hi, uint64_t hi_bytes, const uint8_t* d_lo,
                            uint64_t lo_bytes, const void* d_blob_hi, const void* d_blob_lo,
                            uint32_t chunk, uint64_t n, uint8_t* d_out_hi, uint8_t* d_out_lo,
                            lecb_result* d_res2, void* d_ws, uint64_t ws_bytes, void* stream) {
    const uint8_t* st[2] = {d_hi, d_lo};
    const uint64_t sb[2] = {hi_bytes, lo_bytes};
    const void* bl[2] = {d_blob_hi, d_blob_lo};
    uint8_t* out[2] = {d_out_hi, d_out_lo};
    return decode_common(2, DEC_OUT_PLANES, st, sb, bl, chunk, n, out, nullptr, nullptr, d_res2, d_ws, ws_bytes,
                         stream);
}

int lecb_decode_bf16_planes_from_results(const uint8_t* d_hi, const uint8_t* d_lo,
                                         const lecb_result* d_enc_res2, const void* d_blob_hi,
                                         const void* d_blob_lo, uint32_t chunk, uint64_t n,
                                         uint8_t* d_out_hi, uint8_t* d_out_lo, lecb_result* d_res2,
                                         void* d_ws, uint64_t ws_bytes, void* stream) {
    if (!d_enc_res2) return LECB_ERR_INVALID_ARG;
    const uint8_t* st[2] = {d_hi, d_lo};
    const uint64_t sb[2] = {0, 0};
    const void* bl[2] = {d_blob_hi, d_blob_lo};
    uint8_t* out[2] = {d_out_hi, d_out_lo};
    return decode_common(2, DEC_OUT_PLANES, st, sb, bl, chunk, n, out, nullptr, nullptr, d_res2, d_ws, ws_bytes,
                         stream, d_enc_res2);
}

int lecb_encode_bf16_pertensor(const uint16_t* d_in, uint64_t n, uint32_t chunk,
                               uint32_t max_len, uint64_t* d_hist, void* d_blob_hi,
                               void* d_blob_lo, lecb_codebook* cb_hi, lecb_codebook* cb_lo,
                               uint8_t* d_out_hi, uint64_t cap_hi, uint8_t* d_out_lo,
                               uint64_t cap_lo, lecb_result* d_res2, void* d_ws,
                               uint64_t ws_bytes, void* stream) {
    return pertensor_common(d_in, nullptr, n, chunk, max_len, d_hist, d_blob_hi, d_blob_lo, cb_hi,
                            cb_lo, d_out_hi, cap_hi, d_out_lo, cap_lo, d_res2, d_ws, ws_bytes, stream);
}

int lecb_histogram_bf16_delta(const uint16_t* d_w0, const uint16_t* d_w1, uint64_t n,
                              uint64_t* d_hist_hi, uint64_t* d_hist_lo, int accumulate,
                              void* stream) {
    if (!d_hist_hi || !d_hist_lo || !aligned16(d_hist_hi) || !aligned16(d_hist_lo) ||
        (n && (!d_w0 || !d_w1 || !aligned16(d_w0) || !aligned16(d_w1))))
        return LECB_ERR_INVALID_ARG;
    return launch_histogram_u16(d_w0, d_w1, n, d_hist_hi, d_hist_lo, accumulate, stream);
}

int lecb_encode_bf16_delta(const uint16_t* d_w0, const uint16_t* d_w1, uint64_t n,
                           const void* d_blob_hi, const void* d_blob_lo, uint32_t chunk,
                           uint8_t* d_out_hi, uint64_t cap_hi, uint8_t* d_out_lo, uint64_t cap_lo,
                           lecb_result* d_res2, void* d_ws, uint64_t ws_bytes, void* stream) {
    return encode_common(d_w0, ENC_PAIR_XOR, n, d_blob_hi, chunk, d_out_hi, cap_hi, d_res2, d_ws,
                         ws_bytes, stream, d_blob_lo, d_out_lo, cap_lo, d_w1);
}

int lecb_encode_bf16_delta_pertensor(const uint16_t* d_w0, const uint16_t* d_w1, uint64_t n,
                                     uint32_t chunk, uint32_t max_len, uint64_t* d_hist,
                                     void* d_blob_hi, void* d_blob_lo, lecb_codebook* cb_hi,
                                     lecb_codebook* cb_lo, uint8_t* d_out_hi, uint64_t cap_hi,
                                     uint8_t* d_out_lo, uint64_t cap_lo, lecb_result* d_res2,
                                     void* d_ws, uint64_t ws_bytes, void* stream) {
    if (n && !d_w1) return LECB_ERR_INVALID_ARG;
    return pertensor_common(d_w0, d_w1, n, chunk, max_len, d_hist, d_blob_hi, d_blob_lo, cb_hi,
                            cb_lo, d_out_hi, cap_hi, d_out_lo, cap_lo, d_res2, d_ws, ws_bytes, stream);
}

int lecb_encode_adaptive(const uint8_t* d_in, uint64_t n, uint32_t chunk, uint32_t max_len,
                         uint32_t tol_ppm, uint64_t* d_hist, lecb_codebook* cb, void* d_blob,
                         int* refreshed, uint8_t* d_out, uint64_t cap, lecb_result* d_res,
                         void* d_ws, uint64_t ws_bytes, void* stream) {
    if (!valid_chunk(chunk) || max_len < 1 || max_len > 16 || !d_hist || !aligned16(d_hist) || !cb ||
        !refreshed || !d_res)
        return LECB_ERR_INVALID_ARG;
    *refreshed = 0;
    if (n == 0) return launch_result(d_res, 0, 0, LECB_OK, stream);
    int rc = lecb_histogram(d_in, n, d_hist, 0, stream);
    if (rc) return rc;
    const uint64_t* h = nullptr;
    rc = read_back_hist(d_hist, 256, stream, &h);
    if (rc) return rc;
    rc = lecb_drift_check(h, cb, max_len, tol_ppm, cb, refreshed, nullptr, nullptr);
    if (rc) return rc;
    if (*refreshed) {
        rc = lecb_codebook_upload(cb, d_blob, stream);
        if (rc) return rc;
    }
    return lecb_encode(d_in, n, d_blob, chunk, d_out, cap, d_res, d_ws, ws_bytes, stream);
}

int lecb_decode_bf16(const uint8_t* d_hi, uint64_t hi_bytes, const uint8_t* d_lo,
                     uint64_t lo_bytes, const void* d_blob_hi, const void* d_blob_lo,
                     uint32_t chunk, uint64_t n, uint16_t* d_out,
                     lecb_result* d_res2, void* d_ws, uint64_t ws_bytes, void* stream) {
    if (!d_res2) return LECB_ERR_INVALID_ARG;
    const uint8_t* st[2] = {d_hi, d_lo};
    const uint64_t sb[2] = {hi_bytes, lo_bytes};
    const void* bl[2] = {d_blob_hi, d_blob_lo};
    return decode_common(2, DEC_OUT_U16, st, sb, bl, chunk, n, nullptr, reinterpret_cast<uint8_t*>(d_out), nullptr,
                         d_res2, d_ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- codebooks built on the device

int lecb_build_codebook_device(const uint64_t* d_hist, uint32_t nplanes, uint32_t max_len, uint32_t min_freq,
                               void* const d_blob[], void* stream) {
    if (!d_hist || !aligned16(d_hist) || !d_blob || nplanes < 1 || nplanes > 4 || max_len < 1 || max_len > 16)
        return LECB_ERR_INVALID_ARG;
    const uint64_t* h[4];
    DeviceCodebook* cb[4];
    for (uint32_t p = 0; p < nplanes; ++p) {
        if (!d_blob[p] || !aligned16(d_blob[p])) return LECB_ERR_INVALID_ARG;
        h[p] = d_hist + 256 * p;
        cb[p] = reinterpret_cast<DeviceCodebook*>(d_blob[p]);
    }
    return launch_build_codebooks(h, cb, (int)nplanes, max_len, min_freq, stream);
}

int lecb_codebook_download(const void* d_blob, lecb_codebook* out, void* stream) {
    if (!d_blob || !aligned16(d_blob) || !out) return LECB_ERR_INVALID_ARG;
    uint32_t enc[256];
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(enc, reinterpret_cast<const DeviceCodebook*>(d_blob)->enc, sizeof(enc),
                       hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return LECB_ERR_HIP;
    uint8_t len[256];
    for (int k = 0; k < 256; ++k) len[k] = (uint8_t)(enc[k] & 31u);
    return canonical_from_lengths(len, out);
}

int lecb_pertensor_codebooks(const void* d_in, uint32_t elem_bytes, uint64_t n, uint32_t max_len,
                             uint64_t* d_hist, void* const d_blob[], lecb_codebook cb[], void* stream) {
    if ((elem_bytes != 2 && elem_bytes != 4) || max_len < 1 || max_len > 16 || !d_hist || !aligned16(d_hist) ||
        !d_blob || !cb || n == 0)
        return LECB_ERR_INVALID_ARG;
    const int planes = (int)elem_bytes;
    int rc = elem_bytes == 2
                 ? lecb_histogram_bf16(static_cast<const uint16_t*>(d_in), n, d_hist, d_hist + 256, 0, stream)
                 : lecb_histogram_fp32(static_cast<const uint32_t*>(d_in), n, d_hist, 0, stream);
    if (rc) return rc;
    const uint64_t* h = nullptr;
    rc = read_back_hist(d_hist, 256 * planes, stream, &h);
    for (int p = 0; p < planes && !rc; ++p) rc = lecb_build_codebook(h + 256 * p, max_len, 0, &cb[p]);
    for (int p = 0; p < planes && !rc; ++p) rc = lecb_codebook_upload(&cb[p], d_blob[p], stream);
    return rc;
}

int lecb_encode_bf16_pertensor_nosync(const uint16_t* d_in, uint64_t n, uint32_t chunk, uint32_t max_len,
                                      uint64_t* d_hist, void* d_blob_hi, void* d_blob_lo, uint8_t* d_out_hi,
                                      uint64_t cap_hi, uint8_t* d_out_lo, uint64_t cap_lo, lecb_result* d_res2,
                                      void* d_ws, uint64_t ws_bytes, void* stream) {
    if (!valid_chunk(chunk) || max_len < 1 || max_len > 16 || !d_hist || !aligned16(d_hist) || !d_res2)
        return LECB_ERR_INVALID_ARG;
    if (n == 0) {
        int rc = launch_result(d_res2, 0, 0, LECB_OK, stream);
        return rc ? rc : launch_result(d_res2 + 1, 0, 0, LECB_OK, stream);
    }
    void* blobs[2] = {d_blob_hi, d_blob_lo};
    int rc = lecb_histogram_bf16(d_in, n, d_hist, d_hist + 256, 0, stream);
    if (!rc) rc = lecb_build_codebook_device(d_hist, 2, max_len, 0, blobs, stream);
    if (!rc)
        rc = lecb_encode_bf16(d_in, n, d_blob_hi, d_blob_lo, chunk, d_out_hi, cap_hi, d_out_lo, cap_lo, d_res2,
                              d_ws, ws_bytes, stream);
    return rc;
}

int lecb_encode_bf16_delta_pertensor_nosync(const uint16_t* d_w0, const uint16_t* d_w1, uint64_t n,
                                            uint32_t chunk, uint32_t max_len, uint64_t* d_hist,
                                            void* d_blob_hi, void* d_blob_lo, uint8_t* d_out_hi,
                                            uint64_t cap_hi, uint8_t* d_out_lo, uint64_t cap_lo,
                                            lecb_result* d_res2, void* d_ws, uint64_t ws_bytes, void* stream) {
    if (!valid_chunk(chunk) || max_len < 1 || max_len > 16 || !d_hist || !aligned16(d_hist) || !d_res2)
        return LECB_ERR_INVALID_ARG;
    if (n == 0) {
        int rc = launch_result(d_res2, 0, 0, LECB_OK, stream);
        return rc ? rc : launch_result(d_res2 + 1, 0, 0, LECB_OK, stream);
    }
    void* blobs[2] = {d_blob_hi, d_blob_lo};
    int rc = lecb_histogram_bf16_delta(d_w0, d_w1, n, d_hist, d_hist + 256, 0, stream);
    if (!rc) rc = lecb_build_codebook_device(d_hist, 2, max_len, 0, blobs, stream);
    if (!rc)
        rc = lecb_encode_bf16_delta(d_w0, d_w1, n, d_blob_hi, d_blob_lo, chunk, d_out_hi, cap_hi, d_out_lo, cap_lo,
                                    d_res2, d_ws, ws_bytes, stream);
    return rc;
}

// ---------------------------------------------------------------- 32-bit elements, four planes

int lecb_histogram_fp32(const uint32_t* d_in, uint64_t n, uint64_t* d_hist, int accumulate, void* stream) {
    if (!d_hist || !aligned16(d_hist) || (n && (!d_in || !aligned16(d_in)))) return LECB_ERR_INVALID_ARG;
    return launch_histogram_u32(d_in, n, d_hist, accumulate, stream);
}

int lecb_merge_fp32(const uint8_t* const d_planes[4], uint64_t n, uint32_t* d_out, void* stream) {
    if (!d_planes) return LECB_ERR_INVALID_ARG;
    if (n) {
        if (!d_out || !aligned16(d_out)) return LECB_ERR_INVALID_ARG;
        for (int k = 0; k < 4; ++k)
            if (!d_planes[k] || !aligned16(d_planes[k])) return LECB_ERR_INVALID_ARG;
    }
    return launch_merge4(d_planes[0], d_planes[1], d_planes[2], d_planes[3], n, d_out, stream);
}

int lecb_encode_fp32(const uint32_t* d_in, uint64_t n, const void* const d_blob[4], uint32_t chunk,
                     uint8_t* const d_out[4], const uint64_t cap[4], lecb_result* d_res4, void* d_ws,
                     uint64_t ws_bytes, void* stream) {
    if (!d_blob || !d_out || !cap || !d_res4) return LECB_ERR_INVALID_ARG;
    // bytes 3 and 2 (upper 16 bits), then bytes 1 and 0; the two launches
    // share the workspace one after the other on `stream`
    int rc = encode_common(d_in, ENC_PAIR32_HI, n, d_blob[0], chunk, d_out[0], cap[0], d_res4, d_ws,
                           ws_bytes, stream, d_blob[1], d_out[1], cap[1]);
    if (!rc)
        rc = encode_common(d_in, ENC_PAIR32_LO, n, d_blob[2], chunk, d_out[2], cap[2], d_res4 + 2, d_ws,
                           ws_bytes, stream, d_blob[3], d_out[3], cap[3]);
    return rc;
}

int lecb_encode_fp32_pertensor(const uint32_t* d_in, uint64_t n, uint32_t chunk, uint32_t max_len,
                               uint64_t* d_hist, void* const d_blob[4], lecb_codebook cb[4],
                               uint8_t* const d_out[4], const uint64_t cap[4], lecb_result* d_res4,
                               void* d_ws, uint64_t ws_bytes, void* stream) {
    if (!valid_chunk(chunk) || max_len < 1 || max_len > 16 || !d_hist || !aligned16(d_hist) || !d_blob ||
        !cb || !d_out || !cap || !d_res4)
        return LECB_ERR_INVALID_ARG;
    if (n == 0) {
        for (int k = 0; k < 4; ++k) {
            std::memset(&cb[k], 0, sizeof(cb[k]));
            const int rc = launch_result(d_res4 + k, 0, 0, LECB_OK, stream);
            if (rc) return rc;
        }
        return LECB_OK;
    }
    int rc = lecb_histogram_fp32(d_in, n, d_hist, 0, stream);
    if (rc) return rc;
    const uint64_t* h = nullptr;
    rc = read_back_hist(d_hist, 1024, stream, &h);
    if (rc) return rc;
    for (int k = 0; k < 4 && !rc; ++k) rc = lecb_build_codebook(h + 256 * k, max_len, 0, &cb[k]);
    for (int k = 0; k < 4 && !rc; ++k) rc = lecb_codebook_upload(&cb[k], d_blob[k], stream);
    if (!rc) rc = lecb_encode_fp32(d_in, n, d_blob, chunk, d_out, cap, d_res4, d_ws, ws_bytes, stream);
    return rc;
}

int lecb_encode_fp32_pertensor_nosync(const uint32_t* d_in, uint64_t n, uint32_t chunk, uint32_t max_len,
                                      uint64_t* d_hist, void* const d_blob[4], uint8_t* const d_out[4],
                                      const uint64_t cap[4], lecb_result* d_res4, void* d_ws, uint64_t ws_bytes,
                                      void* stream) {
    if (!valid_chunk(chunk) || max_len < 1 || max_len > 16 || !d_hist || !aligned16(d_hist) || !d_blob ||
        !d_out || !cap || !d_res4)
        return LECB_ERR_INVALID_ARG;
    if (n == 0) {
        for (int k = 0; k < 4; ++k) {
            const int rc = launch_result(d_res4 + k, 0, 0, LECB_OK, stream);
            if (rc) return rc;
        }
        return LECB_OK;
    }
    int rc = lecb_histogram_fp32(d_in, n, d_hist, 0, stream);
    if (!rc) rc = lecb_build_codebook_device(d_hist, 4, max_len, 0, d_blob, stream);
    if (!rc) rc = lecb_encode_fp32(d_in, n, d_blob, chunk, d_out, cap, d_res4, d_ws, ws_bytes, stream);
    return rc;
}

static int decode_fp32_common(const uint8_t* const d_stream[4], const uint64_t* stream_bytes,
                              const lecb_result* d_enc_res4, const void* const d_blob[4], uint32_t chunk,
                              uint64_t n, uint32_t* d_out, lecb_result* d_res4,
                              void* d_ws, uint64_t ws_bytes, void* stream) {
    if (!d_stream || !d_blob || !d_res4 || (!stream_bytes && !d_enc_res4)) return LECB_ERR_INVALID_ARG;
    const uint64_t none[4] = {0, 0, 0, 0};
    return decode_common(4, DEC_OUT_U32, d_stream, stream_bytes ? stream_bytes : none, d_blob, chunk, n, nullptr,
                         reinterpret_cast<uint8_t*>(d_out), nullptr, d_res4, d_ws, ws_bytes, stream, d_enc_res4);
}

int lecb_decode_fp32(const uint8_t* const d_stream[4], const uint64_t stream_bytes[4],
                     const void* const d_blob[4], uint32_t chunk, uint64_t n, uint32_t* d_out,
                     lecb_result* d_res4, void* d_ws, uint64_t ws_bytes, void* stream) {
    if (!stream_bytes) return LECB_ERR_INVALID_ARG;
    return decode_fp32_common(d_stream, stream_bytes, nullptr, d_blob, chunk, n, d_out, d_res4, d_ws, ws_bytes,
                              stream);
}

int lecb_decode_fp32_from_results(const uint8_t* const d_stream[4], const lecb_result* d_enc_res4,
                                  const void* const d_blob[4], uint32_t chunk, uint64_t n, uint32_t* d_out,
                                  lecb_result* d_res4, void* d_ws, uint64_t ws_bytes, void* stream) {
    if (!d_enc_res4) return LECB_ERR_INVALID_ARG;
    return decode_fp32_common(d_stream, nullptr, d_enc_res4, d_blob, chunk, n, d_out, d_res4, d_ws, ws_bytes,
                              stream);
}

}  // extern "C"
