"""Helpers shared by the tests (not collected as tests)."""
import numpy as np

from oracle import codebook as cb

SUB = 256


def string_encode(data, lengths, codes, chunk):
    """Reference container built from '0'/'1' strings (small inputs only)."""
    n = len(data)
    words, cbits, cwo, so = [], [], [0], []
    for c0 in range(0, n, chunk):
        part = data[c0:c0 + chunk]
        bits = ""
        for k, s in enumerate(part):
            if k % SUB == 0:
                so.append(len(bits))
            bits += cb.code_string(codes[s], lengths[s])
        cbits.append(len(bits))
        bits += "0" * (-len(bits) % 32)
        for i in range(0, len(bits), 32):
            words.append(int(bits[i:i + 32], 2))
        cwo.append(len(words))
    return {"payload": np.array(words, dtype=np.uint32), "chunk_bits": np.array(cbits, dtype=np.uint32),
            "chunk_word_offset": np.array(cwo, dtype=np.uint64), "sub_off": np.array(so, dtype=np.uint32)}
