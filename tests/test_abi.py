"""The C-ABI library loads and exports every entry point include/pc.h declares
(no device calls: this runs without a GPU)."""
import ctypes
import os
import re

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pc.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pc_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("pc_codebook_build", "pc_encode", "pc_decode", "pc_num_chunks", "pc_num_substreams",
                 "pc_max_payload_words", "pc_encode_workspace_bytes", "pc_status_string"):
        assert want in names


def test_library_exports_every_declared_symbol():
    import static_codebook_lossless_amd as pc

    lib = ctypes.CDLL(pc.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(pc.EXPORTS) == declared_functions()


def test_binding_has_the_same_names():
    import static_codebook_lossless_amd as pc

    for n in declared_functions():
        if n != "pc_status_string":
            assert hasattr(pc, n), n


def test_status_strings():
    import static_codebook_lossless_amd as pc

    assert pc.status_string(pc.PC_OK) == "ok"
    assert pc.status_string(pc.PC_ERR_CORRUPT) == "corrupt stream"
