"""Python binding of liblecb.so, the MI355X Huffman byte codec.

Argument marshalling only: every step of the coding path runs in the HIP
library.  ``lecb_*`` functions mirror the C ABI in ``include/lecb.h`` one to
one (torch tensors are passed by ``data_ptr()``, the stream is the current
torch stream); the small helpers below them only allocate buffers with torch
and chain those calls.  If the library is not built this module raises on
first use -- there is no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblecb.so")

LECB_OK = 0
LECB_ERR_INVALID_ARG = -1
LECB_ERR_CAPACITY = -2
LECB_ERR_TOO_LARGE = -3
LECB_ERR_NO_SYMBOLS = -4
LECB_ERR_HIP = -5
LECB_ERR_WORKSPACE = -6
LECB_ERR_SCRATCH = -7
LECB_ERR_UNCODED_SYMBOL = -16
LECB_ERR_CORRUPT = -17
CONTAINER_HEADER_BYTES = 560
NOALLOC_SCRATCH_BYTES = 16 << 20


class LecbError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lecb_status_str(status)} ({status})")
        self.status = status


class lecb_codebook(ctypes.Structure):
    _fields_ = [
        ("max_len", ctypes.c_uint32),
        ("num_coded", ctypes.c_uint32),
        ("len", ctypes.c_uint8 * 256),
        ("code", ctypes.c_uint16 * 256),
    ]

    def lengths(self) -> np.ndarray:
        return np.frombuffer(bytes(self.len), dtype=np.uint8).copy()

    def codes(self) -> np.ndarray:
        return np.array(self.code, dtype=np.uint32)


class lecb_stats(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_uint64),
        ("payload_bits", ctypes.c_uint64),
        ("optimal_bits", ctypes.c_uint64),
        ("uncoded", ctypes.c_uint64),
        ("shannon_bits", ctypes.c_double),
    ]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


RESULT_DTYPE = np.dtype([("bytes", "<u8"), ("payload_bits", "<u8"), ("status", "<i4"), ("reserved", "<u4")])

_u64 = ctypes.c_uint64
_u32 = ctypes.c_uint32
_int = ctypes.c_int
_vp = ctypes.c_void_p

_SIGNATURES = {
    "lecb_abi_version": (_u32, []),
    "lecb_status_str": (ctypes.c_char_p, [_int]),
    "lecb_num_chunks": (_u64, [_u64, _u32]),
    "lecb_header_bytes": (_u64, [_u64, _u32]),
    "lecb_encoded_bound": (_u64, [_u64, _u32, _u32]),
    "lecb_workspace_bytes": (_u64, [_u64, _u32]),
    "lecb_build_codebook": (_int, [_vp, _u32, _u32, ctypes.POINTER(lecb_codebook)]),
    "lecb_codebook_from_lengths": (_int, [_vp, ctypes.POINTER(lecb_codebook)]),
    "lecb_device_codebook_bytes": (_u64, []),
    "lecb_stream_stats": (_int, [_vp, _vp, _u32, ctypes.POINTER(lecb_stats)]),
    "lecb_histogram_bf16_delta": (_int, [_vp, _vp, _u64, _vp, _vp, _int, _vp]),
    "lecb_encode_bf16_delta": (_int, [_vp, _vp, _u64, _vp, _vp, _u32, _vp, _u64, _vp, _u64, _vp, _vp, _u64, _vp]),
    "lecb_encode_bf16_delta_pertensor": (_int, [_vp, _vp, _u64, _u32, _u32, _vp, _vp, _vp,
                                                ctypes.POINTER(lecb_codebook), ctypes.POINTER(lecb_codebook),
                                                _vp, _u64, _vp, _u64, _vp, _vp, _u64, _vp]),
    "lecb_decode_bf16_delta": (_int, [_vp, _u64, _vp, _u64, _vp, _vp, _u32, _u64, _vp, _vp, _vp, _vp,
                                      _u64, _vp]),
    "lecb_decode_bf16_delta_from_results": (_int, [_vp, _vp, _vp, _vp, _vp, _u32, _u64, _vp, _vp, _vp,
                                                   _vp, _u64, _vp]),
    "lecb_drift_check": (_int, [_vp, ctypes.POINTER(lecb_codebook), _u32, _u32,
                                ctypes.POINTER(lecb_codebook), ctypes.POINTER(_int),
                                ctypes.POINTER(_u64), ctypes.POINTER(_u64)]),
    "lecb_encode_adaptive": (_int, [_vp, _u64, _u32, _u32, _u32, _vp, ctypes.POINTER(lecb_codebook),
                                    _vp, ctypes.POINTER(_int), _vp, _u64, _vp, _vp, _u64, _vp]),
    "lecb_container_write_header": (_int, [_vp, _u64, _u32, _u32, _vp, _vp, _u64, _u64]),
    "lecb_container_read_header": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "lecb_workspace_init": (_int, [_vp, _u64, _vp]),
    "lecb_codebook_upload": (_int, [ctypes.POINTER(lecb_codebook), _vp, _vp]),
    "lecb_histogram": (_int, [_vp, _u64, _vp, _int, _vp]),
    "lecb_histogram_bf16": (_int, [_vp, _u64, _vp, _vp, _int, _vp]),
    "lecb_split_bf16": (_int, [_vp, _u64, _vp, _vp, _vp]),
    "lecb_merge_bf16": (_int, [_vp, _vp, _u64, _vp, _vp]),
    "lecb_encode": (_int, [_vp, _u64, _vp, _u32, _vp, _u64, _vp, _vp, _u64, _vp]),
    "lecb_decode": (_int, [_vp, _u64, _vp, _u32, _u64, _vp, _vp, _vp, _u64, _vp]),
    "lecb_encode_plane": (_int, [_vp, _u64, _int, _vp, _u32, _vp, _u64, _vp, _vp, _u64, _vp]),
    "lecb_encode_bf16": (_int, [_vp, _u64, _vp, _vp, _u32, _vp, _u64, _vp, _u64, _vp, _vp, _u64, _vp]),
    "lecb_encode_bf16_pertensor": (_int, [_vp, _u64, _u32, _u32, _vp, _vp, _vp,
                                          ctypes.POINTER(lecb_codebook), ctypes.POINTER(lecb_codebook),
                                          _vp, _u64, _vp, _u64, _vp, _vp, _u64, _vp]),
    "lecb_decode_from_result": (_int, [_vp, _vp, _vp, _u32, _u64, _vp, _vp, _vp, _u64, _vp]),
    "lecb_decode_bf16_from_results": (_int, [_vp, _vp, _vp, _vp, _vp, _u32, _u64, _vp, _vp, _vp, _u64, _vp]),
    "lecb_decode_bf16_planes_from_results": (_int, [_vp, _vp, _vp, _vp, _vp, _u32, _u64, _vp, _vp, _vp, _vp,
                                                    _u64, _vp]),
    "lecb_decode_bf16_planes": (_int, [_vp, _u64, _vp, _u64, _vp, _vp, _u32, _u64, _vp, _vp, _vp, _vp, _u64, _vp]),
    "lecb_decode_bf16": (_int, [_vp, _u64, _vp, _u64, _vp, _vp, _u32, _u64, _vp, _vp, _vp, _u64, _vp]),
    "lecb_pertensor_codebooks": (_int, [_vp, _u32, _u64, _u32, _vp, _vp, ctypes.POINTER(lecb_codebook), _vp]),
    "lecb_build_codebook_device": (_int, [_vp, _u32, _u32, _u32, _vp, _vp]),
    "lecb_codebook_download": (_int, [_vp, ctypes.POINTER(lecb_codebook), _vp]),
    "lecb_encode_bf16_pertensor_nosync": (_int, [_vp, _u64, _u32, _u32, _vp, _vp, _vp, _vp, _u64, _vp, _u64,
                                                 _vp, _vp, _u64, _vp]),
    "lecb_encode_bf16_delta_pertensor_nosync": (_int, [_vp, _vp, _u64, _u32, _u32, _vp, _vp, _vp, _vp, _u64,
                                                       _vp, _u64, _vp, _vp, _u64, _vp]),
    "lecb_encode_fp32_pertensor_nosync": (_int, [_vp, _u64, _u32, _u32, _vp, _vp, _vp, _vp, _vp, _vp, _u64,
                                                 _vp]),
    "lecb_encode_noalloc": (_int, [_vp, _u64, _vp, _u32, _vp, _u64, _vp, _vp]),
    "lecb_histogram_fp32": (_int, [_vp, _u64, _vp, _int, _vp]),
    "lecb_merge_fp32": (_int, [_vp, _u64, _vp, _vp]),
    "lecb_encode_fp32": (_int, [_vp, _u64, _vp, _u32, _vp, _vp, _vp, _vp, _u64, _vp]),
    "lecb_encode_fp32_pertensor": (_int, [_vp, _u64, _u32, _u32, _vp, _vp, ctypes.POINTER(lecb_codebook),
                                          _vp, _vp, _vp, _vp, _u64, _vp]),
    "lecb_decode_fp32": (_int, [_vp, _vp, _vp, _u32, _u64, _vp, _vp, _vp, _u64, _vp]),
    "lecb_decode_fp32_from_results": (_int, [_vp, _vp, _vp, _u32, _u64, _vp, _vp, _vp, _u64, _vp]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load liblecb.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch first: the library's HIP runtime dependency must resolve to the
        # runtime torch already holds, or the process ends up with two runtimes
        # and the second one finds no device
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m lossless_entropy_coding_byte_amd.build`"
            )
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols() -> list[str]:
    return list(_SIGNATURES)


def _check(rc: int, where: str) -> None:
    if rc != LECB_OK:
        raise LecbError(rc, where)


def _stream(stream=None):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


# --------------------------------------------------------------------------- host functions

def lecb_abi_version() -> int:
    return load().lecb_abi_version()


def lecb_status_str(status: int) -> str:
    return load().lecb_status_str(status).decode()


def lecb_num_chunks(n: int, chunk: int) -> int:
    return load().lecb_num_chunks(n, chunk)


def lecb_header_bytes(n: int, chunk: int) -> int:
    return load().lecb_header_bytes(n, chunk)


def lecb_encoded_bound(n: int, chunk: int, max_len: int = 16) -> int:
    return load().lecb_encoded_bound(n, chunk, max_len)


def lecb_workspace_bytes(n: int, chunk: int) -> int:
    return load().lecb_workspace_bytes(n, chunk)


def lecb_device_codebook_bytes() -> int:
    return load().lecb_device_codebook_bytes()


def lecb_build_codebook(hist, max_len: int = 16, min_freq: int = 1) -> lecb_codebook:
    h = np.ascontiguousarray(np.asarray(hist, dtype=np.uint64))
    if h.shape != (256,):
        raise ValueError("histogram must have 256 bins")
    cb = lecb_codebook()
    _check(load().lecb_build_codebook(h.ctypes.data, max_len, min_freq, ctypes.byref(cb)),
           "lecb_build_codebook")
    return cb


def lecb_codebook_from_lengths(lengths) -> lecb_codebook:
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.uint8))
    if ln.shape != (256,):
        raise ValueError("lengths must have 256 entries")
    cb = lecb_codebook()
    _check(load().lecb_codebook_from_lengths(ln.ctypes.data, ctypes.byref(cb)),
           "lecb_codebook_from_lengths")
    return cb


def lecb_stream_stats(hist, lengths, max_len: int = 16) -> dict:
    h = np.ascontiguousarray(np.asarray(hist, dtype=np.uint64))
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.uint8))
    if h.shape != (256,) or ln.shape != (256,):
        raise ValueError("histogram and lengths must have 256 entries")
    st = lecb_stats()
    _check(load().lecb_stream_stats(h.ctypes.data, ln.ctypes.data, max_len, ctypes.byref(st)),
           "lecb_stream_stats")
    return st.as_dict()


def lecb_drift_check(hist, cur: lecb_codebook, max_len: int = 16, tol_ppm: int = 0):
    """Refresh decision for one batch: (refreshed, codebook to use, bits_cur or None, bits_opt)."""
    h = np.ascontiguousarray(np.asarray(hist, dtype=np.uint64))
    if h.shape != (256,):
        raise ValueError("histogram must have 256 bins")
    out = lecb_codebook()
    ref = _int(0)
    bc, bo = _u64(0), _u64(0)
    _check(load().lecb_drift_check(h.ctypes.data, ctypes.byref(cur), max_len, tol_ppm, ctypes.byref(out),
                                   ctypes.byref(ref), ctypes.byref(bc), ctypes.byref(bo)),
           "lecb_drift_check")
    return bool(ref.value), out, (None if bc.value == 2**64 - 1 else int(bc.value)), int(bo.value)


def lecb_container_write_header(n, chunk, max_len, len_hi, len_lo, bytes_hi, bytes_lo) -> np.ndarray:
    out = np.zeros(CONTAINER_HEADER_BYTES, np.uint8)
    hi = np.ascontiguousarray(len_hi, dtype=np.uint8)
    lo = np.ascontiguousarray(len_lo, dtype=np.uint8)
    _check(load().lecb_container_write_header(out.ctypes.data, n, chunk, max_len, hi.ctypes.data,
                                              lo.ctypes.data, bytes_hi, bytes_lo),
           "lecb_container_write_header")
    return out


def lecb_container_read_header(buf) -> dict:
    b = np.ascontiguousarray(np.asarray(buf, dtype=np.uint8)[:CONTAINER_HEADER_BYTES])
    n, bh, bl = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    chunk, ml = ctypes.c_uint32(), ctypes.c_uint32()
    hi = np.zeros(256, np.uint8)
    lo = np.zeros(256, np.uint8)
    _check(load().lecb_container_read_header(b.ctypes.data, ctypes.byref(n), ctypes.byref(chunk),
                                             ctypes.byref(ml), hi.ctypes.data, lo.ctypes.data,
                                             ctypes.byref(bh), ctypes.byref(bl)),
           "lecb_container_read_header")
    return {"n": n.value, "chunk": chunk.value, "max_len": ml.value, "len_hi": hi, "len_lo": lo,
            "bytes_hi": bh.value, "bytes_lo": bl.value}


# --------------------------------------------------------------------------- device functions

def lecb_workspace_init(ws, stream=None) -> None:
    _check(load().lecb_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "lecb_workspace_init")


def lecb_codebook_upload(cb: lecb_codebook, blob, stream=None) -> None:
    _check(load().lecb_codebook_upload(ctypes.byref(cb), _ptr(blob), _stream(stream)),
           "lecb_codebook_upload")


def lecb_histogram(x, hist, accumulate: bool = False, stream=None) -> None:
    _check(load().lecb_histogram(_ptr(x), x.numel() * x.element_size(), _ptr(hist), int(accumulate),
                                 _stream(stream)), "lecb_histogram")


def lecb_histogram_bf16(x, hist_hi, hist_lo, accumulate: bool = False, stream=None) -> None:
    _check(load().lecb_histogram_bf16(_ptr(x), x.numel(), _ptr(hist_hi), _ptr(hist_lo),
                                      int(accumulate), _stream(stream)), "lecb_histogram_bf16")


def lecb_split_bf16(x, hi, lo, stream=None) -> None:
    _check(load().lecb_split_bf16(_ptr(x), x.numel(), _ptr(hi), _ptr(lo), _stream(stream)),
           "lecb_split_bf16")


def lecb_merge_bf16(hi, lo, out, stream=None) -> None:
    _check(load().lecb_merge_bf16(_ptr(hi), _ptr(lo), out.numel(), _ptr(out), _stream(stream)),
           "lecb_merge_bf16")


def lecb_encode(x, n, blob, chunk, out, res, ws, stream=None) -> None:
    _check(load().lecb_encode(_ptr(x), n, _ptr(blob), chunk, _ptr(out), out.numel(), _ptr(res),
                              _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "lecb_encode")


def lecb_encode_noalloc(x, n, blob, chunk, out, res, stream=None) -> None:
    _check(load().lecb_encode_noalloc(_ptr(x), n, _ptr(blob), chunk, _ptr(out), out.numel(), _ptr(res),
                                      _stream(stream)),
           "lecb_encode_noalloc")


def lecb_encode_plane(x, n, plane, blob, chunk, out, res, ws, stream=None) -> None:
    _check(load().lecb_encode_plane(_ptr(x), n, plane, _ptr(blob), chunk, _ptr(out), out.numel(),
                                    _ptr(res), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)), "lecb_encode_plane")


def lecb_encode_bf16(x, n, blob_hi, blob_lo, chunk, out_hi, out_lo, res2, ws, stream=None) -> None:
    """Both byte planes of 16-bit words in one pass; res2 holds two results (hi, lo)."""
    _check(load().lecb_encode_bf16(_ptr(x), n, _ptr(blob_hi), _ptr(blob_lo), chunk, _ptr(out_hi),
                                   out_hi.numel(), _ptr(out_lo), out_lo.numel(), _ptr(res2),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "lecb_encode_bf16")


def lecb_decode_from_result(stream_buf, enc_res, blob, chunk, n, out, res, ws, stream=None) -> None:
    """Decode with the stream size read on the device from the encoder's result."""
    _check(load().lecb_decode_from_result(_ptr(stream_buf), _ptr(enc_res), _ptr(blob), chunk, n,
                                          _ptr(out), _ptr(res), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)),
           "lecb_decode_from_result")


def lecb_decode_bf16_from_results(hi, lo, enc_res2, blob_hi, blob_lo, chunk, n, out, res2, ws,
                                  stream=None) -> None:
    """Both planes decoded into the 16-bit words, sizes read on the device from the encoder's results."""
    _check(load().lecb_decode_bf16_from_results(_ptr(hi), _ptr(lo), _ptr(enc_res2), _ptr(blob_hi),
                                                _ptr(blob_lo), chunk, n, _ptr(out),
                                                _ptr(res2), _ptr(ws), ws.numel() * ws.element_size(),
                                                _stream(stream)),
           "lecb_decode_bf16_from_results")


def lecb_decode_bf16_planes(hi, hi_bytes, lo, lo_bytes, blob_hi, blob_lo, chunk, n, out_hi, out_lo,
                            res2, ws, stream=None) -> None:
    """Both byte planes decoded in one launch into two byte tensors."""
    _check(load().lecb_decode_bf16_planes(_ptr(hi), hi_bytes, _ptr(lo), lo_bytes, _ptr(blob_hi),
                                          _ptr(blob_lo), chunk, n, _ptr(out_hi), _ptr(out_lo),
                                          _ptr(res2), _ptr(ws), ws.numel() * ws.element_size(),
                                          _stream(stream)),
           "lecb_decode_bf16_planes")


def lecb_decode_bf16_planes_from_results(hi, lo, enc_res2, blob_hi, blob_lo, chunk, n, out_hi, out_lo, res2, ws,
                                         stream=None) -> None:
    """Both byte planes decoded in one launch, sizes read on the device from the encoder's results."""
    _check(load().lecb_decode_bf16_planes_from_results(_ptr(hi), _ptr(lo), _ptr(enc_res2), _ptr(blob_hi),
                                                       _ptr(blob_lo), chunk, n, _ptr(out_hi), _ptr(out_lo),
                                                       _ptr(res2), _ptr(ws), ws.numel() * ws.element_size(),
                                                       _stream(stream)),
           "lecb_decode_bf16_planes_from_results")


def lecb_decode(stream_buf, stream_bytes, blob, chunk, n, out, res, ws, stream=None) -> None:
    _check(load().lecb_decode(_ptr(stream_buf), stream_bytes, _ptr(blob), chunk, n, _ptr(out),
                              _ptr(res), _ptr(ws), ws.numel() * ws.element_size(),
                              _stream(stream)), "lecb_decode")


def lecb_encode_bf16_pertensor(x, n, chunk, max_len, hist, blob_hi, blob_lo, out_hi, out_lo,
                               res2, ws, stream=None):
    cb_hi, cb_lo = lecb_codebook(), lecb_codebook()
    _check(load().lecb_encode_bf16_pertensor(
        _ptr(x), n, chunk, max_len, _ptr(hist), _ptr(blob_hi), _ptr(blob_lo), ctypes.byref(cb_hi),
        ctypes.byref(cb_lo), _ptr(out_hi), out_hi.numel(), _ptr(out_lo), out_lo.numel(),
        _ptr(res2), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "lecb_encode_bf16_pertensor")
    return cb_hi, cb_lo


def lecb_histogram_bf16_delta(w0, w1, hist_hi, hist_lo, accumulate: bool = False, stream=None) -> None:
    """Histograms of the byte planes of w0 ^ w1."""
    _check(load().lecb_histogram_bf16_delta(_ptr(w0), _ptr(w1), w0.numel(), _ptr(hist_hi), _ptr(hist_lo),
                                            int(accumulate), _stream(stream)), "lecb_histogram_bf16_delta")


def lecb_encode_bf16_delta(w0, w1, n, blob_hi, blob_lo, chunk, out_hi, out_lo, res2, ws, stream=None) -> None:
    _check(load().lecb_encode_bf16_delta(_ptr(w0), _ptr(w1), n, _ptr(blob_hi), _ptr(blob_lo), chunk,
                                         _ptr(out_hi), out_hi.numel(), _ptr(out_lo), out_lo.numel(),
                                         _ptr(res2), _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream(stream)), "lecb_encode_bf16_delta")


def lecb_encode_bf16_delta_pertensor(w0, w1, n, chunk, max_len, hist, blob_hi, blob_lo, out_hi, out_lo,
                                     res2, ws, stream=None):
    cb_hi, cb_lo = lecb_codebook(), lecb_codebook()
    _check(load().lecb_encode_bf16_delta_pertensor(
        _ptr(w0), _ptr(w1), n, chunk, max_len, _ptr(hist), _ptr(blob_hi), _ptr(blob_lo), ctypes.byref(cb_hi),
        ctypes.byref(cb_lo), _ptr(out_hi), out_hi.numel(), _ptr(out_lo), out_lo.numel(),
        _ptr(res2), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "lecb_encode_bf16_delta_pertensor")
    return cb_hi, cb_lo


def lecb_decode_bf16_delta(hi, hi_bytes, lo, lo_bytes, blob_hi, blob_lo, chunk, n, w0, w1, res2,
                           ws, stream=None) -> None:
    _check(load().lecb_decode_bf16_delta(_ptr(hi), hi_bytes, _ptr(lo), lo_bytes, _ptr(blob_hi),
                                         _ptr(blob_lo), chunk, n, _ptr(w0), _ptr(w1),
                                         _ptr(res2), _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream(stream)), "lecb_decode_bf16_delta")


def lecb_decode_bf16_delta_from_results(hi, lo, enc_res2, blob_hi, blob_lo, chunk, n, w0, w1,
                                        res2, ws, stream=None) -> None:
    _check(load().lecb_decode_bf16_delta_from_results(
        _ptr(hi), _ptr(lo), _ptr(enc_res2), _ptr(blob_hi), _ptr(blob_lo), chunk, n, _ptr(w0), _ptr(w1),
        _ptr(res2), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "lecb_decode_bf16_delta_from_results")


def lecb_encode_adaptive(x, n, chunk, max_len, tol_ppm, hist, cb: lecb_codebook, blob, out, res, ws,
                         stream=None) -> bool:
    """One batch of a drifting stream; cb is updated in place.  Returns whether it was refreshed."""
    ref = _int(0)
    _check(load().lecb_encode_adaptive(_ptr(x), n, chunk, max_len, tol_ppm, _ptr(hist), ctypes.byref(cb),
                                       _ptr(blob), ctypes.byref(ref), _ptr(out), out.numel(), _ptr(res),
                                       _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "lecb_encode_adaptive")
    return bool(ref.value)


def lecb_decode_bf16(hi, hi_bytes, lo, lo_bytes, blob_hi, blob_lo, chunk, n, out, res2, ws,
                     stream=None) -> None:
    _check(load().lecb_decode_bf16(_ptr(hi), hi_bytes, _ptr(lo), lo_bytes, _ptr(blob_hi),
                                   _ptr(blob_lo), chunk, n, _ptr(out), _ptr(res2),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "lecb_decode_bf16")


# --------------------------------------------------------------------------- codebooks built on the device

def lecb_build_codebook_device(hist, blobs, max_len: int = 16, min_freq: int = 0, stream=None) -> None:
    """Codebook of each 256-bin histogram in hist (int64[256 * len(blobs)]) into the device blobs."""
    ptrs = (ctypes.c_void_p * len(blobs))(*[b.data_ptr() for b in blobs])
    _check(load().lecb_build_codebook_device(_ptr(hist), len(blobs), max_len, min_freq, ptrs, _stream(stream)),
           "lecb_build_codebook_device")


def lecb_pertensor_codebooks(x, n, max_len, hist, blobs, stream=None) -> list:
    """Plane histograms -> read back -> host codebooks -> upload; x is int16 (bf16) or int32 (fp32)."""
    eb = x.element_size()
    cbs = (lecb_codebook * eb)()
    ptrs = (ctypes.c_void_p * len(blobs))(*[b.data_ptr() for b in blobs])
    if len(blobs) != eb:
        raise ValueError("one codebook blob per byte plane")
    _check(load().lecb_pertensor_codebooks(_ptr(x), eb, n, max_len, _ptr(hist), ptrs, cbs, _stream(stream)),
           "lecb_pertensor_codebooks")
    return list(cbs)


def lecb_codebook_download(blob, stream=None) -> lecb_codebook:
    cb = lecb_codebook()
    _check(load().lecb_codebook_download(_ptr(blob), ctypes.byref(cb), _stream(stream)), "lecb_codebook_download")
    return cb


def lecb_encode_bf16_pertensor_nosync(x, n, chunk, max_len, hist, blob_hi, blob_lo, out_hi, out_lo, res2, ws,
                                      stream=None) -> None:
    _check(load().lecb_encode_bf16_pertensor_nosync(
        _ptr(x), n, chunk, max_len, _ptr(hist), _ptr(blob_hi), _ptr(blob_lo), _ptr(out_hi), out_hi.numel(),
        _ptr(out_lo), out_lo.numel(), _ptr(res2), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "lecb_encode_bf16_pertensor_nosync")


def lecb_encode_bf16_delta_pertensor_nosync(w0, w1, n, chunk, max_len, hist, blob_hi, blob_lo, out_hi, out_lo,
                                            res2, ws, stream=None) -> None:
    _check(load().lecb_encode_bf16_delta_pertensor_nosync(
        _ptr(w0), _ptr(w1), n, chunk, max_len, _ptr(hist), _ptr(blob_hi), _ptr(blob_lo), _ptr(out_hi),
        out_hi.numel(), _ptr(out_lo), out_lo.numel(), _ptr(res2), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)), "lecb_encode_bf16_delta_pertensor_nosync")


def lecb_encode_fp32_pertensor_nosync(x, n, chunk, max_len, hist, blobs, outs, res4, ws, stream=None) -> None:
    _check(load().lecb_encode_fp32_pertensor_nosync(_ptr(x), n, chunk, max_len, _ptr(hist), _ptrs4(blobs),
                                                    _ptrs4(outs), _caps4(outs), _ptr(res4), _ptr(ws),
                                                    ws.numel() * ws.element_size(), _stream(stream)),
           "lecb_encode_fp32_pertensor_nosync")


# --------------------------------------------------------------------------- 32-bit elements, four planes
# Per-plane lists are in plane order: byte 3 (sign, high exponent bits) first.

def _ptrs4(ts):
    if len(ts) != 4:
        raise ValueError("four planes expected")
    return (ctypes.c_void_p * 4)(*[t.data_ptr() for t in ts])


def _caps4(ts):
    return (_u64 * 4)(*[t.numel() for t in ts])


def lecb_histogram_fp32(x, hist, accumulate: bool = False, stream=None) -> None:
    """Histograms of the four byte planes of 32-bit elements into hist (int64[1024])."""
    _check(load().lecb_histogram_fp32(_ptr(x), x.numel(), _ptr(hist), int(accumulate), _stream(stream)),
           "lecb_histogram_fp32")


def lecb_merge_fp32(planes, out, stream=None) -> None:
    _check(load().lecb_merge_fp32(_ptrs4(planes), out.numel(), _ptr(out), _stream(stream)), "lecb_merge_fp32")


def lecb_encode_fp32(x, n, blobs, chunk, outs, res4, ws, stream=None) -> None:
    _check(load().lecb_encode_fp32(_ptr(x), n, _ptrs4(blobs), chunk, _ptrs4(outs), _caps4(outs), _ptr(res4),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "lecb_encode_fp32")


def lecb_encode_fp32_pertensor(x, n, chunk, max_len, hist, blobs, outs, res4, ws, stream=None):
    """Per-tensor four-plane encode; returns the four host codebooks."""
    cbs = (lecb_codebook * 4)()
    _check(load().lecb_encode_fp32_pertensor(_ptr(x), n, chunk, max_len, _ptr(hist), _ptrs4(blobs), cbs,
                                             _ptrs4(outs), _caps4(outs), _ptr(res4), _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(stream)),
           "lecb_encode_fp32_pertensor")
    return list(cbs)


def lecb_decode_fp32(streams, stream_bytes, blobs, chunk, n, out, res4, ws, stream=None) -> None:
    sb = (_u64 * 4)(*[int(b) for b in stream_bytes])
    _check(load().lecb_decode_fp32(_ptrs4(streams), sb, _ptrs4(blobs), chunk, n, _ptr(out),
                                   _ptr(res4), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "lecb_decode_fp32")


def lecb_decode_fp32_from_results(streams, enc_res4, blobs, chunk, n, out, res4, ws,
                                  stream=None) -> None:
    _check(load().lecb_decode_fp32_from_results(_ptrs4(streams), _ptr(enc_res4), _ptrs4(blobs), chunk, n,
                                                _ptr(out), _ptr(res4), _ptr(ws),
                                                ws.numel() * ws.element_size(), _stream(stream)),
           "lecb_decode_fp32_from_results")


# --------------------------------------------------------------------------- buffer helpers

def results_to_numpy(res) -> np.ndarray:
    """Copy lecb_result structs from device memory (synchronises with the copy)."""
    return res.cpu().numpy().view(RESULT_DTYPE)


def new_results(count: int, device):
    import torch

    return torch.zeros(count * RESULT_DTYPE.itemsize, dtype=torch.uint8, device=device)


def new_codebook_blob(device):
    import torch

    return torch.zeros(lecb_device_codebook_bytes(), dtype=torch.uint8, device=device)


def new_workspace(n: int, chunk: int, device):
    import torch

    ws = torch.empty(lecb_workspace_bytes(n, chunk), dtype=torch.uint8, device=device)
    lecb_workspace_init(ws)
    return ws


@dataclass
class DeviceCodebook:
    """A canonical codebook and its device-resident tables."""

    codebook: lecb_codebook
    blob: object

    @classmethod
    def upload(cls, cb: lecb_codebook, device) -> "DeviceCodebook":
        blob = new_codebook_blob(device)
        lecb_codebook_upload(cb, blob)
        return cls(cb, blob)


def encode_bytes(x, dcb: DeviceCodebook, chunk: int, ws=None, out=None, res=None):
    """Encode a uint8 device tensor; returns (stream buffer, result tensor)."""
    import torch

    n = x.numel()
    out = out if out is not None else torch.empty(max(16, lecb_encoded_bound(n, chunk)), dtype=torch.uint8, device=x.device)
    res = res if res is not None else new_results(1, x.device)
    ws = ws if ws is not None else new_workspace(n, chunk, x.device)
    lecb_encode(x, n, dcb.blob, chunk, out, res, ws)
    return out, res


def decode_bytes(stream_buf, stream_bytes: int, dcb: DeviceCodebook, chunk: int, n: int, ws=None,
                 out=None, res=None):
    import torch

    dev = stream_buf.device
    out = out if out is not None else torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    res = res if res is not None else new_results(1, dev)
    ws = ws if ws is not None else new_workspace(n, chunk, dev)
    lecb_decode(stream_buf, stream_bytes, dcb.blob, chunk, n, out, res, ws)
    return out, res


# --------------------------------------------------------------------------- tensor-level helpers

def encode(x, dcb: DeviceCodebook, chunk: int):
    """Fixed-codebook encode of a uint8 device tensor: (stream buffer, result tensor)."""
    return encode_bytes(x, dcb, chunk)


def decode(stream_buf, stream_bytes: int, dcb: DeviceCodebook, chunk: int, n: int):
    """Decode a stream back to n bytes: (uint8 tensor, result tensor)."""
    return decode_bytes(stream_buf, stream_bytes, dcb, chunk, n)


def encode_bf16(x, chunk: int, max_len: int = 16) -> np.ndarray:
    """Per-tensor coding of a 16-bit tensor on its device, written as the container
    (header with both plane codebooks' lengths, then both streams) in host memory.

    The codebooks are built on the device; the host reads the two results and
    lengths once, to size and label the container."""
    import torch

    dev = x.device
    xv = x.contiguous().view(torch.int16).view(-1)
    n = xv.numel()
    cap = max(16, lecb_encoded_bound(n, chunk, max_len))
    hist = torch.zeros(512, dtype=torch.int64, device=dev)
    bh, bl = new_codebook_blob(dev), new_codebook_blob(dev)
    oh = torch.empty(cap, dtype=torch.uint8, device=dev)
    ol = torch.empty(cap, dtype=torch.uint8, device=dev)
    res = new_results(2, dev)
    ws = new_workspace(n, chunk, dev)
    if n:
        lecb_encode_bf16_pertensor_nosync(xv, n, chunk, max_len, hist, bh, bl, oh, ol, res, ws)
    r = results_to_numpy(res)
    for k in range(2):
        if int(r[k]["status"]) != LECB_OK:
            raise LecbError(int(r[k]["status"]), "encode_bf16")
    len_hi = lecb_codebook_download(bh).lengths() if n else np.zeros(256, np.uint8)
    len_lo = lecb_codebook_download(bl).lengths() if n else np.zeros(256, np.uint8)
    sh, sl = int(r[0]["bytes"]), int(r[1]["bytes"])
    head = lecb_container_write_header(n, chunk, max_len, len_hi, len_lo, sh, sl)
    pad = (-sh) % 16
    return np.concatenate([head, oh[:sh].cpu().numpy(), np.zeros(pad, np.uint8), ol[:sl].cpu().numpy()])


def decode_bf16(container, device):
    """Decode a container written by encode_bf16 into a 16-bit tensor (int16 view) on device."""
    import torch

    buf = np.ascontiguousarray(np.asarray(container, dtype=np.uint8))
    h = lecb_container_read_header(buf)
    n, chunk, sh, sl = h["n"], h["chunk"], h["bytes_hi"], h["bytes_lo"]
    out = torch.empty(max(n, 1), dtype=torch.int16, device=device)
    if n == 0:
        return out[:0]
    off_lo = CONTAINER_HEADER_BYTES + sh + (-sh) % 16
    if buf.size != off_lo + sl:
        raise LecbError(LECB_ERR_CORRUPT, "decode_bf16: container size")
    dh = torch.zeros(sh + 16, dtype=torch.uint8, device=device)
    dl = torch.zeros(sl + 16, dtype=torch.uint8, device=device)
    dh[:sh] = torch.from_numpy(buf[CONTAINER_HEADER_BYTES:CONTAINER_HEADER_BYTES + sh]).to(device)
    dl[:sl] = torch.from_numpy(buf[off_lo:off_lo + sl]).to(device)
    ch = DeviceCodebook.upload(lecb_codebook_from_lengths(h["len_hi"]), device)
    cl = DeviceCodebook.upload(lecb_codebook_from_lengths(h["len_lo"]), device)
    res = new_results(2, device)
    ws = new_workspace(n, chunk, device)
    lecb_decode_bf16(dh, sh, dl, sl, ch.blob, cl.blob, chunk, n, out, res, ws)
    r = results_to_numpy(res)
    for k in range(2):
        if int(r[k]["status"]) != LECB_OK:
            raise LecbError(int(r[k]["status"]), "decode_bf16")
    return out
