"""Fixed-codebook ("single-stage") prefix coding of 8-bit tensors on MI355X.

The work happens in libpc.so (HIP kernels for gfx950 behind a C ABI declared
in include/pc.h); this package only binds it.  Import fails if the library
has not been built.
"""
from ._lib import (  # noqa: F401
    CODEBOOK_BYTES, EXPORTS, LIB_PATH, PC_CODEBOOK_HUFFMAN, PC_CODEBOOK_QLC, PC_ERR_CAPACITY, PC_ERR_CORRUPT,
    PC_ERR_HIP, PC_ERR_INVALID_ARG, PC_ERR_TIMEOUT, PC_ERR_UNSUPPORTED, PC_OK, Encoded, PcError, alloc_encode_outputs,
    codebook_fields, pc_codebook_build, pc_codebook_fit, pc_codebook_validate, pc_decode, pc_decode_qlc, pc_encode,
    pc_encode_noalloc, pc_encode_set_wait_limit, pc_encode_workspace_bytes, pc_histogram, pc_max_payload_words,
    pc_num_chunks, pc_num_substreams, pc_qlc_optimal_bits, pc_shard_code_lengths, pc_traffic_probe, status_string,
)
from .refresh import CodebookRefresh  # noqa: F401,E402
