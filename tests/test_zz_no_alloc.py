"""pc_encode_noalloc (the encode entry point that allocates nothing on the
device) against pc_encode, through the C ABI, on two calls in a row: the
second with a smaller input, so stale workspace contents of the first would
show.  Element by element: payload words, chunk bits, chunk word offsets,
side index and status."""
import ctypes as C
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _encode_both(pc, dcb, x, chunk):
    """(pc_encode's outputs, pc_encode_noalloc's outputs) as host arrays."""
    lib = pc._lib.lib
    n = x.numel()
    res = []
    for which in ("pc_encode", "pc_encode_noalloc"):
        payload, bits, cwo, sub, ws, status = pc.alloc_encode_outputs(n, chunk, x.device)
        for t in (payload, bits, cwo, sub, status):
            t.fill_(-1)  # stale contents: anything not written shows
        torch.cuda.synchronize()
        stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
        p = [C.c_void_p(t.data_ptr()) for t in (dcb, x, payload, bits, cwo, sub, ws, status)]
        if which == "pc_encode":
            st = lib.pc_encode(p[0], p[1], n, chunk, p[2], payload.numel(), p[3], p[4], p[5], p[6], ws.numel() * 8,
                               p[7], stream)
        else:
            st = lib.pc_encode_noalloc(p[0], p[1], n, chunk, p[2], payload.numel(), p[3], p[4], p[5], p[7], stream)
        assert st == pc.PC_OK, (which, st)
        torch.cuda.synchronize()
        nc = pc.pc_num_chunks(n, chunk)
        cwo_h = cwo.cpu().numpy().view(np.uint64)
        res.append({
            "status": int(status.item()),
            "chunk_word_offset": cwo_h,
            "payload": payload[: int(cwo_h[nc])].cpu().numpy().view(np.uint32),
            "chunk_bits": bits[:nc].cpu().numpy().view(np.uint32),
            "sub_off": sub[: pc.pc_num_substreams(n, chunk)].cpu().numpy().view(np.uint32),
        })
    return res


def test_noalloc_matches_pc_encode_twice_shrinking():
    import static_codebook_lossless_amd as pc

    cases = [("ffn1_act", W.WORKLOADS["ffn1_act"].chunk), ("normal_1m", W.WORKLOADS["normal_1m"].chunk)]
    for name, chunk in cases:  # 64 MiB in 4096 chunks, then 1 MiB in 256 chunks
        x_np = W.make(name, 0)
        counts = np.bincount(W.make(name, 1), minlength=256).astype(np.uint64)
        dcb = pc.pc_codebook_build(counts).to(DEV)
        x = torch.from_numpy(x_np).to(DEV)
        say("noalloc vs pc_encode:", name, x_np.size, "bytes, chunk", chunk)
        ref, got = _encode_both(pc, dcb, x, chunk)
        assert ref["status"] == pc.PC_OK and got["status"] == pc.PC_OK
        for k in ("chunk_word_offset", "chunk_bits", "sub_off", "payload"):
            a, b = got[k], ref[k]
            assert a.shape == b.shape, (name, k)
            if not np.array_equal(a, b):
                i = int(np.flatnonzero(a != b)[0])
                raise AssertionError("%s %s differs first at %d" % (name, k, i))
        # and it still decodes
        enc = pc.Encoded(torch.from_numpy(got["payload"].view(np.int32).copy()).to(DEV),
                         torch.from_numpy(got["chunk_bits"].view(np.int32).copy()).to(DEV),
                         torch.from_numpy(got["chunk_word_offset"].view(np.int64).copy()).to(DEV),
                         torch.from_numpy(got["sub_off"].view(np.int32).copy()).to(DEV), x_np.size, chunk)
        out, status = pc.pc_decode(dcb, enc)
        torch.cuda.synchronize()
        assert int(status.item()) == 0 and torch.equal(out, x)


def test_noalloc_rejects_more_chunks_than_its_array():
    import static_codebook_lossless_amd as pc

    lib = pc._lib.lib
    a = C.c_void_p(1 << 20)  # never dereferenced: the size check comes first
    n, chunk = ((1 << 20) + 1) * 256, 256
    st = lib.pc_encode_noalloc(a, a, n, chunk, a, pc.pc_max_payload_words(n, chunk), a, a, a, a, None)
    assert st == pc.PC_ERR_CAPACITY
    n = (1 << 20) * 256  # exactly at the limit: passes the checks (not launched here)
    assert pc.pc_num_chunks(n, chunk) == 1 << 20
