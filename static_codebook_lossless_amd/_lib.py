"""Thin ctypes binding of libpc.so.

Argument marshalling only: torch tensors supply device memory, the current
torch stream supplies the HIP stream, and every step of encoding and decoding
runs in the library's HIP kernels.  There is no fallback: if libpc.so has not
been built, importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import NamedTuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpc.so")

PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED, PC_ERR_CAPACITY, PC_ERR_CORRUPT, PC_ERR_HIP, PC_ERR_TIMEOUT = range(7)
PC_CODEBOOK_HUFFMAN, PC_CODEBOOK_QLC = 0, 1
CODEBOOK_BYTES = 9536
SUBSTREAM = 256

EXPORTS = [
    "pc_status_string", "pc_codebook_build", "pc_codebook_validate", "pc_qlc_optimal_bits", "pc_codebook_fit",
    "pc_shard_code_lengths",
    "pc_num_chunks", "pc_num_substreams", "pc_max_payload_words", "pc_encode_workspace_bytes",
    "pc_encode", "pc_encode_noalloc", "pc_encode_set_wait_limit", "pc_decode", "pc_decode_qlc", "pc_histogram",
    "pc_traffic_probe",
]


class PcError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s: %s (status %d)" % (what, status_string(status), status))
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libpc.so is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                          "or `python static_codebook_lossless_amd/build.py`")
    lib = C.CDLL(LIB_PATH)
    p, sz, i = C.c_void_p, C.c_size_t, C.c_int
    lib.pc_status_string.argtypes = [i]
    lib.pc_status_string.restype = C.c_char_p
    lib.pc_codebook_build.argtypes = [p, i, p, p]
    lib.pc_codebook_validate.argtypes = [p]
    lib.pc_qlc_optimal_bits.argtypes = [p, p]
    lib.pc_codebook_fit.argtypes = [p, p, p, p]
    lib.pc_shard_code_lengths.argtypes = [p, p]
    for f in ("pc_num_chunks", "pc_num_substreams", "pc_max_payload_words", "pc_encode_workspace_bytes"):
        getattr(lib, f).argtypes = [sz, sz]
        getattr(lib, f).restype = sz
    lib.pc_encode.argtypes = [p, p, sz, sz, p, sz, p, p, p, p, sz, p, p]
    lib.pc_encode_noalloc.argtypes = [p, p, sz, sz, p, sz, p, p, p, p, p]
    lib.pc_encode_set_wait_limit.argtypes = [C.c_uint32]
    lib.pc_encode_set_wait_limit.restype = C.c_uint32
    lib.pc_decode.argtypes = [p, p, sz, p, p, p, sz, sz, p, p, p]
    lib.pc_decode_qlc.argtypes = [p, p, sz, p, p, p, sz, sz, p, p, p]
    lib.pc_histogram.argtypes = [p, sz, p, p]
    lib.pc_traffic_probe.argtypes = [p, p, sz, p]
    for f in ("pc_codebook_build", "pc_codebook_validate", "pc_qlc_optimal_bits", "pc_codebook_fit",
              "pc_shard_code_lengths", "pc_encode", "pc_encode_noalloc",
              "pc_decode", "pc_decode_qlc", "pc_histogram", "pc_traffic_probe"):
        getattr(lib, f).restype = i
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.pc_status_string(int(status)).decode()


def _check(status, what):
    if status != PC_OK:
        raise PcError(status, what)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return C.c_void_p(t.ctypes.data)
    return C.c_void_p(t.data_ptr())


def _stream(device):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _counts_u64(counts) -> np.ndarray:
    a = np.asarray(counts.cpu() if isinstance(counts, torch.Tensor) else counts)
    if a.shape != (256,):
        raise ValueError("counts must have 256 entries")
    if a.dtype == np.int64:
        a = a.view(np.uint64)
    return np.ascontiguousarray(a.astype(np.uint64, copy=False))


# ---------------------------------------------------------------------------
# host entry points
# ---------------------------------------------------------------------------

def pc_codebook_build(counts, kind="huffman", qlc_bits=None) -> torch.Tensor:
    """Build the fixed codebook on the host; returns its 9536-byte blob (CPU uint8)."""
    k = {"huffman": PC_CODEBOOK_HUFFMAN, "qlc": PC_CODEBOOK_QLC}.get(kind, kind)
    cnt = _counts_u64(counts)
    bits = None
    if qlc_bits is not None:
        bits = np.ascontiguousarray(np.asarray(qlc_bits, dtype=np.uint8))
        if bits.shape != (8,):
            raise ValueError("qlc_bits must have 8 entries")
    out = torch.zeros(CODEBOOK_BYTES, dtype=torch.uint8)
    _check(lib.pc_codebook_build(_ptr(cnt), int(k), _ptr(bits), _ptr(out)), "pc_codebook_build")
    return out


def pc_codebook_validate(cb: torch.Tensor) -> None:
    cb = cb.cpu().contiguous()
    _check(lib.pc_codebook_validate(_ptr(cb)), "pc_codebook_validate")


def pc_qlc_optimal_bits(counts) -> tuple:
    cnt = _counts_u64(counts)
    out = np.zeros(8, dtype=np.uint8)
    _check(lib.pc_qlc_optimal_bits(_ptr(cnt), _ptr(out)), "pc_qlc_optimal_bits")
    return tuple(int(v) for v in out)


def pc_codebook_fit(cb: torch.Tensor, counts) -> tuple:
    """(bits per symbol the codebook spends on a batch with these counts, the batch's entropy)."""
    cb = cb.cpu().contiguous()
    cnt = _counts_u64(counts)
    avg, ent = C.c_double(), C.c_double()
    _check(lib.pc_codebook_fit(_ptr(cb), _ptr(cnt), C.byref(avg), C.byref(ent)), "pc_codebook_fit")
    return avg.value, ent.value


def pc_shard_code_lengths(counts) -> np.ndarray:
    """Lengths (uint8 [256], 0 = no codeword) of the per-shard comparator code
    built on ``counts`` alone, absent byte values excluded."""
    cnt = _counts_u64(counts)
    out = np.zeros(256, dtype=np.uint8)
    _check(lib.pc_shard_code_lengths(_ptr(cnt), _ptr(out)), "pc_shard_code_lengths")
    return out


def pc_num_chunks(n, chunk):
    return int(lib.pc_num_chunks(n, chunk))


def pc_num_substreams(n, chunk):
    return int(lib.pc_num_substreams(n, chunk))


def pc_max_payload_words(n, chunk):
    return int(lib.pc_max_payload_words(n, chunk))


def pc_encode_workspace_bytes(n, chunk):
    return int(lib.pc_encode_workspace_bytes(n, chunk))


def codebook_fields(cb: torch.Tensor) -> dict:
    """Decode the blob's header and arrays (host view, for tests and reports)."""
    b = cb.cpu().numpy()
    hdr = b[:32].view(np.uint32)
    return {
        "magic": int(hdr[0]), "version": int(hdr[1]), "kind": int(hdr[2]), "max_len": int(hdr[3]),
        "codebook_id": int(hdr[4]), "complete": int(hdr[5]),
        "length": b[32:288].copy(), "code": b[288:800].view(np.uint16).copy(),
        "dec_sym": b[800:4896].copy(), "dec_len": b[4896:8992].copy(),
        "qlc_bits": b[8992:9000].copy(), "qlc_start": b[9000:9016].view(np.uint16).copy(),
        "rank_of": b[9016:9272].copy(), "sym_of_rank": b[9272:9528].copy(),
    }


# ---------------------------------------------------------------------------
# device entry points
# ---------------------------------------------------------------------------

class Encoded(NamedTuple):
    payload: torch.Tensor            # int32 words (raw bits; view as uint32)
    chunk_bits: torch.Tensor         # int32 [num_chunks]
    chunk_word_offset: torch.Tensor  # int64 [num_chunks + 1]
    sub_off: torch.Tensor            # int32 [num_substreams]
    n: int
    chunk: int
    status: torch.Tensor | None = None  # int32 [1]: PC_OK, or PC_ERR_TIMEOUT (outputs invalid)


def alloc_encode_outputs(n, chunk, device):
    """(payload, chunk_bits, chunk_word_offset, sub_off, workspace, status) device buffers."""
    nc = pc_num_chunks(n, chunk)
    payload = torch.empty(max(pc_max_payload_words(n, chunk), 4), dtype=torch.int32, device=device)
    chunk_bits = torch.empty(max(nc, 1), dtype=torch.int32, device=device)
    cwo = torch.empty(nc + 1, dtype=torch.int64, device=device)
    sub_off = torch.empty(max(pc_num_substreams(n, chunk), 1), dtype=torch.int32, device=device)
    ws = torch.empty(max(pc_encode_workspace_bytes(n, chunk) // 8, 1), dtype=torch.int64, device=device)
    status = torch.empty(1, dtype=torch.int32, device=device)
    return payload, chunk_bits, cwo, sub_off, ws, status


def pc_encode_set_wait_limit(polls: int) -> int:
    """Set the encoder's bounded-wait limit (polls; 0 = the default); returns the previous one."""
    return int(lib.pc_encode_set_wait_limit(int(polls)))


def pc_encode(d_cb: torch.Tensor, d_in: torch.Tensor, chunk: int, outputs=None) -> Encoded:
    """Encode the uint8 device tensor ``d_in``.  ``outputs`` (from
    ``alloc_encode_outputs``) may be passed to reuse buffers.  Asynchronous
    on the current stream; ``payload`` is the full-capacity buffer, its first
    ``chunk_word_offset[-1]`` words are the stream.  ``status`` (device) reads
    PC_OK after the stream has run the call, unless the device-side wait gave
    up (PC_ERR_TIMEOUT: the outputs are then invalid)."""
    if d_in.dtype != torch.uint8 or not d_in.is_cuda:
        raise TypeError("d_in must be a uint8 CUDA tensor")
    x = d_in.reshape(-1)
    n = x.numel()
    payload, chunk_bits, cwo, sub_off, ws, status = outputs or alloc_encode_outputs(n, chunk, x.device)
    st = lib.pc_encode(_ptr(d_cb), _ptr(x), n, chunk, _ptr(payload), payload.numel(), _ptr(chunk_bits),
                       _ptr(cwo), _ptr(sub_off), _ptr(ws), ws.numel() * 8, _ptr(status), _stream(x.device))
    _check(st, "pc_encode")
    nc = pc_num_chunks(n, chunk)
    return Encoded(payload, chunk_bits[:nc], cwo, sub_off[:pc_num_substreams(n, chunk)], n, chunk, status)


def pc_encode_noalloc(d_cb: torch.Tensor, d_in: torch.Tensor, chunk: int, outputs=None) -> Encoded:
    """``pc_encode`` through the entry point that allocates nothing on the
    device: its workspace is the library's own static array (at most 2^20
    chunks; calls that overlap on one GPU race).  The workspace entry of
    ``outputs`` is not used."""
    if d_in.dtype != torch.uint8 or not d_in.is_cuda:
        raise TypeError("d_in must be a uint8 CUDA tensor")
    x = d_in.reshape(-1)
    n = x.numel()
    payload, chunk_bits, cwo, sub_off, _, status = outputs or alloc_encode_outputs(n, chunk, x.device)
    st = lib.pc_encode_noalloc(_ptr(d_cb), _ptr(x), n, chunk, _ptr(payload), payload.numel(), _ptr(chunk_bits),
                               _ptr(cwo), _ptr(sub_off), _ptr(status), _stream(x.device))
    _check(st, "pc_encode_noalloc")
    nc = pc_num_chunks(n, chunk)
    return Encoded(payload, chunk_bits[:nc], cwo, sub_off[:pc_num_substreams(n, chunk)], n, chunk, status)


def _decode(fn, name, d_cb, enc: Encoded, payload_words=None, out=None, status=None):
    n, chunk = enc.n, enc.chunk
    dev = enc.payload.device
    if out is None:
        out = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    if payload_words is None:
        payload_words = enc.payload.numel()
    st = fn(_ptr(d_cb), _ptr(enc.payload), int(payload_words), _ptr(enc.chunk_bits), _ptr(enc.chunk_word_offset),
            _ptr(enc.sub_off), n, chunk, _ptr(out), _ptr(status), _stream(dev))
    _check(st, name)
    return out[:n], status


def pc_decode(d_cb, enc: Encoded, payload_words=None, out=None, status=None):
    """Decode ``enc`` with the generic 12-bit-peek engine.  Returns
    (bytes, status tensor); the caller reads status after synchronising.
    ``status`` must be zero on entry when passed in."""
    return _decode(lib.pc_decode, "pc_decode", d_cb, enc, payload_words, out, status)


def pc_decode_qlc(d_cb, enc: Encoded, payload_words=None, out=None, status=None):
    """Decode a QLC stream with the area/index decoder of "Quad Length Codes for
    Lossless Compression of e4m3" (abstract)."""
    return _decode(lib.pc_decode_qlc, "pc_decode_qlc", d_cb, enc, payload_words, out, status)


def pc_histogram(d_in: torch.Tensor, counts: torch.Tensor | None = None) -> torch.Tensor:
    """Accumulate the byte histogram of ``d_in`` into ``counts`` (int64 [256] on the device)."""
    x = d_in.reshape(-1)
    if counts is None:
        counts = torch.zeros(256, dtype=torch.int64, device=x.device)
    _check(lib.pc_histogram(_ptr(x), x.numel(), _ptr(counts), _stream(x.device)), "pc_histogram")
    return counts


def pc_traffic_probe(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Copy ``src`` into ``dst`` (same byte size, a multiple of 16) with the
    coder kernels' 16-byte non-temporal loads and stores: a known transfer
    for calibrating hardware traffic counters."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not (src.is_cuda and dst.is_cuda):
        raise ValueError("pc_traffic_probe: src and dst must be device tensors of the same byte size")
    _check(lib.pc_traffic_probe(_ptr(src), _ptr(dst), nbytes, _stream(src.device)), "pc_traffic_probe")
