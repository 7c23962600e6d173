"""lecb_encode_noalloc (the encode for callers that cannot allocate): the
same stream and result as lecb_encode, on two calls in a row with the second
input smaller, and a clear error for an input beyond its static scratch."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import lossless_entropy_coding_byte_amd as lecb
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


def _codebook():
    warm = np.sum([oracle.histogram(workloads.int8_fixed(r, 1 << 18)) for r in (1, 2)], axis=0, dtype=np.uint64)
    return lecb.DeviceCodebook.upload(lecb.lecb_build_codebook(warm, 16, 1), DEV)


def test_noalloc_equals_encode_on_two_calls():
    dcb = _codebook()
    for n, chunk, seed in ((3_000_001, 4096, 1), (777_777, 16384, 2)):  # the second call is smaller
        print(f"[noalloc] n={n} chunk={chunk}", flush=True)
        x = workloads.q8(np.random.default_rng([200, seed]).normal(0.0, 20.0, n))
        xd = torch.from_numpy(x).to(DEV)
        cap = lecb.lecb_encoded_bound(n, chunk)
        ref = torch.zeros(cap, dtype=torch.uint8, device=DEV)
        got = torch.full((cap,), 0xA5, dtype=torch.uint8, device=DEV)
        rr, rg = lecb.new_results(1, DEV), lecb.new_results(1, DEV)
        lecb.lecb_encode(xd, n, dcb.blob, chunk, ref, rr, lecb.new_workspace(n, chunk, DEV))
        lecb.lecb_encode_noalloc(xd, n, dcb.blob, chunk, got, rg)
        a, b = lecb.results_to_numpy(rr)[0], lecb.results_to_numpy(rg)[0]
        assert int(a["status"]) == 0 and int(b["status"]) == 0
        assert int(a["bytes"]) == int(b["bytes"]) and int(a["payload_bits"]) == int(b["payload_bits"])
        nb = int(a["bytes"])
        assert torch.equal(ref[:nb], got[:nb])


def test_noalloc_rejects_inputs_beyond_its_scratch():
    dcb = _codebook()
    chunk = 256   # 4 Mi chunks: their workspace (8 bytes per chunk and stream) is over 16 MiB
    n = 1 << 30
    assert lecb.lecb_workspace_bytes(n, chunk) > lecb.NOALLOC_SCRATCH_BYTES
    buf = torch.zeros(1024, dtype=torch.uint8, device=DEV)
    res = lecb.new_results(1, DEV)
    with pytest.raises(lecb.LecbError) as e:
        lecb.lecb_encode_noalloc(buf, n, dcb.blob, chunk, buf, res)
    assert e.value.status == lecb.LECB_ERR_SCRATCH
    assert "scratch" in lecb.lecb_status_str(lecb.LECB_ERR_SCRATCH)
