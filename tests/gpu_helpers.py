"""Shared helpers of the GPU tests: run the HIP path through the C ABI, compare with the oracle."""

import numpy as np
import torch

import oracle
import lossless_entropy_coding_byte_amd as lecb

DEV = "cuda:0"


def to_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def codebook_for(x: np.ndarray, clamp: bool, max_len: int = 16):
    h = oracle.histogram(x)
    F = oracle.codebook_frequencies([h], 1 if clamp else 0)
    return oracle.package_merge_lengths(F, max_len)


def gpu_encode(x: np.ndarray, lengths: np.ndarray, chunk: int):
    """Encode host bytes on the GPU; returns (stream bytes as numpy, result record, device codebook)."""
    cb = lecb.lecb_codebook_from_lengths(lengths)
    dcb = lecb.DeviceCodebook.upload(cb, DEV)
    xd = to_dev(x) if x.size else torch.empty(16, dtype=torch.uint8, device=DEV)
    out, res = lecb.encode_bytes(xd, dcb, chunk) if x.size else _empty_encode(dcb, chunk)
    r = lecb.results_to_numpy(res)[0]
    nbytes = int(r["bytes"])
    return out[:nbytes].cpu().numpy(), r, dcb


def _empty_encode(dcb, chunk):
    out = torch.zeros(16, dtype=torch.uint8, device=DEV)
    res = lecb.new_results(1, DEV)
    ws = lecb.new_workspace(0, chunk, DEV)
    lecb.lecb_encode(out, 0, dcb.blob, chunk, out, res, ws)
    return out, res


def gpu_decode(stream: np.ndarray, dcb, chunk: int, n: int):
    buf = torch.zeros((stream.size + 15) // 16 * 16 + 16, dtype=torch.uint8, device=DEV)
    if stream.size:
        buf[: stream.size] = to_dev(stream)
    out, res = lecb.decode_bytes(buf, stream.size, dcb, chunk, n)
    r = lecb.results_to_numpy(res)[0]
    return out[:n].cpu().numpy(), r
