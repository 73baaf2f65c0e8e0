"""Argument checks of the device entry points, on the CPU: every call here
is rejected before the library touches the device (fake, never dereferenced
addresses), so no GPU is needed."""
import ctypes as C

import pytest

import static_codebook_lossless_amd as pc

lib = pc._lib.lib
P = C.c_void_p
A = P(1 << 20)      # 16-byte aligned fake device address
ODD = P((1 << 20) + 4)  # 4-byte aligned only
CHUNK = 65536


def enc(cb=A, x=A, n=1000, chunk=CHUNK, payload=A, cap=None, bits=A, cwo=A, sub=A, ws=A, ws_bytes=None,
        status=A):
    cap = pc.pc_max_payload_words(n, chunk) if cap is None else cap
    ws_bytes = pc.pc_encode_workspace_bytes(n, chunk) if ws_bytes is None else ws_bytes
    return lib.pc_encode(cb, x, n, chunk, payload, cap, bits, cwo, sub, ws, ws_bytes, status, None)


def dec(fn, cb=A, payload=A, words=100, bits=A, cwo=A, sub=A, n=1000, chunk=CHUNK, out=A, status=A):
    return fn(cb, payload, words, bits, cwo, sub, n, chunk, out, status, None)


@pytest.mark.parametrize("chunk", [0, 1, 255, 257, 1000, (1 << 24) + 256, 1 << 25])
def test_bad_chunk_sizes(chunk):
    assert enc(chunk=chunk, cap=1 << 30, ws_bytes=1 << 30) == pc.PC_ERR_INVALID_ARG
    for fn in (lib.pc_decode, lib.pc_decode_qlc):
        assert dec(fn, chunk=chunk) == pc.PC_ERR_INVALID_ARG
    assert pc.pc_num_chunks(1000, chunk) == 0 and pc.pc_max_payload_words(1000, chunk) == 0
    assert pc.pc_encode_workspace_bytes(1000, chunk) == 0


@pytest.mark.parametrize("which", ["cb", "x", "payload", "bits", "cwo", "sub", "ws", "status"])
def test_encode_null_pointers(which):
    assert enc(**{which: None}) == pc.PC_ERR_INVALID_ARG


@pytest.mark.parametrize("which", ["cb", "x", "payload", "cwo", "ws"])
def test_encode_misaligned_pointers(which):
    assert enc(**{which: ODD}) == pc.PC_ERR_INVALID_ARG
    assert enc(status=P((1 << 20) + 2)) == pc.PC_ERR_INVALID_ARG


def test_encode_wait_limit_round_trips():
    prev = pc.pc_encode_set_wait_limit(7)
    try:
        assert pc.pc_encode_set_wait_limit(0) == 7
        assert pc.pc_encode_set_wait_limit(0) == prev  # 0 restores the default
    finally:
        pc.pc_encode_set_wait_limit(prev)


def test_encode_capacity():
    assert enc(cap=pc.pc_max_payload_words(1000, CHUNK) - 1) == pc.PC_ERR_CAPACITY
    assert enc(ws_bytes=pc.pc_encode_workspace_bytes(1000, CHUNK) - 1) == pc.PC_ERR_CAPACITY


@pytest.mark.parametrize("which", ["cb", "payload", "bits", "cwo", "sub", "out", "status"])
def test_decode_null_pointers(which):
    for fn in (lib.pc_decode, lib.pc_decode_qlc):
        assert dec(fn, **{which: None}) == pc.PC_ERR_INVALID_ARG


@pytest.mark.parametrize("which", ["cb", "payload", "out"])
def test_decode_misaligned_pointers(which):
    for fn in (lib.pc_decode, lib.pc_decode_qlc):
        assert dec(fn, **{which: ODD}) == pc.PC_ERR_INVALID_ARG


def test_empty_decode_and_histogram_touch_nothing():
    for fn in (lib.pc_decode, lib.pc_decode_qlc):
        assert dec(fn, cb=None, payload=None, bits=None, cwo=None, sub=None, out=None, status=None, n=0) == pc.PC_OK
    assert lib.pc_histogram(None, 0, None, None) == pc.PC_OK
    assert lib.pc_histogram(None, 10, A, None) == pc.PC_ERR_INVALID_ARG
    assert lib.pc_histogram(A, 10, ODD, None) == pc.PC_ERR_INVALID_ARG


def test_size_limits():
    # the largest sizes each entry point serves, checked before any device
    # access: encode up to 2^31 - 1 chunks, decode below 2^32 - 256 sub-streams
    big = 1 << 46
    assert enc(n=big, chunk=256, cap=1 << 62, ws_bytes=1 << 62) == pc.PC_ERR_UNSUPPORTED
    for fn in (lib.pc_decode, lib.pc_decode_qlc):
        assert dec(fn, n=(0xFFFFFF00) * 256, chunk=1 << 24) == pc.PC_ERR_UNSUPPORTED
        assert dec(fn, n=big) == pc.PC_ERR_UNSUPPORTED


def test_traffic_probe_args():
    assert lib.pc_traffic_probe(None, None, 0, None) == pc.PC_OK
    assert lib.pc_traffic_probe(None, A, 64, None) == pc.PC_ERR_INVALID_ARG
    assert lib.pc_traffic_probe(A, None, 64, None) == pc.PC_ERR_INVALID_ARG
    assert lib.pc_traffic_probe(A, A, 63, None) == pc.PC_ERR_INVALID_ARG
    assert lib.pc_traffic_probe(ODD, A, 64, None) == pc.PC_ERR_INVALID_ARG


def test_workspace_of_multi_unit_chunks():
    # chunks of several 64 KiB units keep one u32 per unit of the full chunks
    for n, chunk in ((1 << 30, 1 << 17), ((1 << 30) + 5000, 1 << 20), (3 << 24, 1 << 24)):
        nc = pc.pc_num_chunks(n, chunk)
        units = (n // chunk) * (chunk // 65536)
        assert pc.pc_encode_workspace_bytes(n, chunk) == 8 * (1 + nc) + 8 * ((units + 1) // 2)
    assert pc.pc_encode_workspace_bytes(1 << 30, 65536) == 8 * (1 + (1 << 14))
    assert pc.pc_encode_workspace_bytes(1 << 30, 3 * 65536 // 2) == 8 * (1 + pc.pc_num_chunks(1 << 30, 98304))


def test_noalloc_rejects_a_workspace_beyond_its_array():
    # 2^37 bytes in 16 MiB chunks: 8192 chunks, but 2^21 unit counts
    n, chunk = 1 << 37, 1 << 24
    cap = pc.pc_max_payload_words(n, chunk)
    assert lib.pc_encode_noalloc(A, A, n, chunk, A, cap, A, A, A, A, None) == pc.PC_ERR_CAPACITY
