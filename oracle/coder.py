"""ctypes front end of the oracle's bit-serial C coder -- TEST INFRASTRUCTURE ONLY.

Container and corruption rules are stated in ``coder.c``.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

OK, INVALID_ARG, CAPACITY, CORRUPT = 0, 1, 3, 4
SUB = 256

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = C.CDLL(_build.LIB)
        p = C.c_void_p
        u64 = C.c_uint64
        lib.oracle_encode.argtypes = [p, u64, u64, p, p, p, u64, p, p, p, C.c_int]
        lib.oracle_encode.restype = C.c_int
        lib.oracle_decode.argtypes = [p, u64, p, p, p, u64, u64, p, C.c_int, p, p, p, C.c_int]
        lib.oracle_decode.restype = C.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return C.c_void_p(a.ctypes.data) if a.size else C.c_void_p(0)


def num_chunks(n, chunk):
    return -(-n // chunk)


def num_substreams(n, chunk):
    nc = num_chunks(n, chunk)
    if nc == 0:
        return 0
    last = n - (nc - 1) * chunk
    return (nc - 1) * (chunk // SUB) + -(-last // SUB)


def max_payload_words(n, chunk):
    nc = num_chunks(n, chunk)
    if nc == 0:
        return 0
    last = n - (nc - 1) * chunk
    return (nc - 1) * (-(-(12 * chunk) // 32)) + -(-(12 * last) // 32)


def encode(data, lengths, codes, chunk, threads=1):
    """Bit-serial encode.  Returns dict(payload, chunk_bits, chunk_word_offset, sub_off)."""
    lib = _load()
    x = np.ascontiguousarray(np.asarray(data, dtype=np.uint8).reshape(-1))
    n = x.size
    nc = num_chunks(n, chunk)
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.uint8))
    cd = np.ascontiguousarray(np.asarray(codes, dtype=np.uint16))
    cap = max(max_payload_words(n, chunk), 1)
    payload = np.zeros(cap, dtype=np.uint32)
    cbits = np.zeros(max(nc, 1), dtype=np.uint32)
    cwo = np.zeros(nc + 1, dtype=np.uint64)
    so = np.zeros(max(num_substreams(n, chunk), 1), dtype=np.uint32)
    rc = lib.oracle_encode(_ptr(x), n, chunk, _ptr(ln), _ptr(cd), _ptr(payload), cap,
                           _ptr(cbits), _ptr(cwo), _ptr(so), int(threads))
    if rc != OK:
        raise ValueError("oracle_encode failed with status %d" % rc)
    total = int(cwo[nc])
    return {
        "payload": payload[:total].copy(),
        "chunk_bits": cbits[:nc].copy(),
        "chunk_word_offset": cwo,
        "sub_off": so[:num_substreams(n, chunk)].copy(),
    }


def decode(streams, n, chunk, codebook, threads=1):
    """Bit-serial decode.  Returns (bytes, status)."""
    lib = _load()
    payload = np.ascontiguousarray(np.asarray(streams["payload"], dtype=np.uint32))
    cbits = np.ascontiguousarray(np.asarray(streams["chunk_bits"], dtype=np.uint32))
    cwo = np.ascontiguousarray(np.asarray(streams["chunk_word_offset"], dtype=np.uint64))
    so = np.ascontiguousarray(np.asarray(streams["sub_off"], dtype=np.uint32))
    out = np.zeros(max(n, 1), dtype=np.uint8)
    ln = np.ascontiguousarray(np.asarray(codebook["lengths"], dtype=np.uint8))
    qlc = 1 if codebook["kind"] == "qlc" else 0
    qb = np.zeros(8, dtype=np.uint8)
    sor = np.zeros(256, dtype=np.uint8)
    if qlc:
        qb[:] = codebook["qlc_bits"]
        sor[:] = codebook["sym_of_rank"]
    if num_chunks(n, chunk) and cwo.size < num_chunks(n, chunk) + 1:
        return out[:n], CORRUPT
    rc = lib.oracle_decode(_ptr(payload), payload.size, _ptr(cbits), _ptr(cwo), _ptr(so), n, chunk,
                           _ptr(ln), qlc, _ptr(qb), _ptr(sor), _ptr(out), int(threads))
    return out[:n], rc
