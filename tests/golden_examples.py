"""Parser for tests/golden/worked_examples.txt (hand-derived examples)."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.txt")


def _pairs(text, base):
    out = {}
    for tok in text.split():
        k, v = tok.split(":")
        out[int(k, 16)] = v if base is None else int(v, base)
    return out


def _hex_bytes(text):
    """Hex byte tokens; "xx*k" is k bytes of value xx."""
    out = []
    for tok in text.split():
        v, _, k = tok.partition("*")
        out += [int(v, 16)] * (int(k) if k else 1)
    return np.array(out, np.uint8)


def load():
    blocks, cur = [], {}
    with open(GOLDEN) as f:
        for raw in f:
            line = raw.strip()
            if line.startswith("#"):
                continue
            if not line:
                if cur:
                    blocks.append(cur)
                    cur = {}
                continue
            key, val = line.split(":", 1)
            cur[key.strip()] = val.strip()
    if cur:
        blocks.append(cur)
    examples = []
    for b in blocks:
        ex = {"name": b["name"], "max_len": int(b["max_len"])}
        freq = np.zeros(256, np.uint64)
        for s, v in _pairs(b["freq"], 10).items():
            freq[s] = v
        ex["freq"] = freq
        ln = np.zeros(256, np.uint8)
        for s, v in _pairs(b["lengths"], 10).items():
            ln[s] = v
        ex["lengths"] = ln
        ex["codes"] = _pairs(b["codes"], None)  # sym -> bit string
        if "input" in b:
            ex["chunk"] = int(b["chunk"])
            ex["input"] = _hex_bytes(b["input"])
            ex["stream"] = _hex_bytes(b["stream"])
            ex["payload_bits"] = int(b["payload_bits"])
        examples.append(ex)
    return examples


CONTAINER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "container_header.txt")


def load_container():
    """The hand-derived container header: its fields and its 560 bytes."""
    fields, head = {}, np.zeros(560, np.uint8)
    with open(CONTAINER) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            key = key.strip()
            if key.isdigit():
                b = [int(t, 16) for t in val.split()]
                head[int(key):int(key) + len(b)] = b
            elif key in ("len_hi", "len_lo"):
                ln = np.zeros(256, np.uint8)
                for s, v in _pairs(val, 10).items():
                    ln[s] = v
                fields[key] = ln
            else:
                fields[key] = int(val)
    return fields, head
