"""Seeded synthetic 8-bit tensors shaped like the workloads the pages discuss.

This module only *generates inputs*.  It holds none of the coder's arithmetic
(no histogram, no code construction, no bit packing): the oracle and the HIP
path both receive the bytes it produces.

The pages measure on real tensors (Gemma 2B activations and weights on
"Single-Stage Huffman Encoder for ML Compression", abstract; e4m3 FFN1/FFN2
activations on "Quad Length Codes for Lossless Compression of e4m3",
Figures 1 and 4; LLM weights on "Huff-LLM", abstract).  None of those tensors
is available, so every workload here is a seeded stand-in with the same
element type and shape.

Recipes (all fp32 draws come from numpy's PCG64 ``default_rng``):

* ``e4m3``: scale a float32 tensor so that its largest magnitude maps to 448
  (the largest finite OCP E4M3FN value), clip to +-448, then cast with
  round-to-nearest-even (torch ``float8_e4m3fn``).  Bytes 0x7F/0xFF (NaN)
  never occur; negative values that round to zero become 0x80 (-0).
* ``int8``: per output row, scale = absmax/127, ``q = clip(rint(w/scale),
  -127, 127)`` stored as two's complement (0x80 never occurs).

Workload ids follow the five configurations of the benchmark:

1. ``normal_1m``:   2**20 e4m3 of N(0,1).
2. ``ffn1_act``:    4096 x 16384 e4m3, row r scaled by s_r ~ LogNormal(0, 0.5).
3. ``gelu_act``:    4096 x 16384 e4m3 of GELU_erf(N(0,1)).
4. ``int8_weight``: 11008 x 4096 int8 of N(0, 0.02), per-row absmax quantized.
5. ``stream_1g``:   16 segments of 2**26 e4m3, segment k ~ N(0, sigma_k),
   sigma_k ~ U(0.5, 2), each segment scaled to absmax 448 on its own.

A "previous batch" is the same recipe under another seed (seed 1 for one
batch, seeds 1..8 for the eight batches of ``ffn1_act``).  Segmented
generators draw each segment from ``default_rng(SeedSequence([seed, k]))`` so
that segments can be generated in parallel threads and independently of each
other; the scalar draws (row scales, segment sigmas) come from
``default_rng(seed)``.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass

import numpy as np

__all__ = [
    "WORKLOADS",
    "Workload",
    "e4m3_from_f32",
    "make",
    "make_previous",
    "num_segments",
]

E4M3_MAX = 448.0


def e4m3_from_f32(x: np.ndarray) -> np.ndarray:
    """Scale ``x`` to absmax 448 and cast to OCP E4M3FN bytes (RNE, saturating)."""
    import torch

    x = np.asarray(x, dtype=np.float32)
    m = float(np.abs(x).max()) if x.size else 0.0
    if m == 0.0:
        return np.zeros(x.shape, dtype=np.uint8).reshape(-1)
    scale = np.float32(E4M3_MAX) / np.float32(m)
    y = x * scale
    np.clip(y, -E4M3_MAX, E4M3_MAX, out=y)
    t = torch.from_numpy(np.ascontiguousarray(y).reshape(-1))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _int8_rows(w: np.ndarray) -> np.ndarray:
    absmax = np.abs(w).max(axis=1, keepdims=True).astype(np.float32)
    absmax[absmax == 0] = 1.0
    scale = absmax / np.float32(127.0)
    q = np.rint(w / scale)
    np.clip(q, -127, 127, out=q)
    return q.astype(np.int8).view(np.uint8).reshape(-1)


def _gelu_erf(x: np.ndarray) -> np.ndarray:
    import torch

    return torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()


def _seg_rng(seed: int, k: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(k)]))


@dataclass(frozen=True)
class Workload:
    name: str
    n: int                 # symbols (bytes)
    chunk: int             # chunk size in symbols
    kind: str              # "huffman" or "qlc"
    qlc_bits: tuple | None  # index widths of the 8 QLC areas
    prev_seeds: tuple      # seeds of the previous batches the codebook is built from
    segments: int          # number of independently generated segments
    description: str


WORKLOADS = {
    "normal_1m": Workload(
        "normal_1m", 1 << 20, 4096, "huffman", None, (1,), 1,
        "2^20 e4m3 of N(0,1); Huffman-12 codebook from a seed-1 batch; 4 KiB chunks"),
    "ffn1_act": Workload(
        "ffn1_act", 4096 * 16384, 16384, "huffman", None, tuple(range(1, 9)), 16,
        "4096x16384 e4m3 FFN1-like activation, rows scaled by LogNormal(0,0.5); "
        "Huffman-12 from the pooled histogram of 8 previous batches; 16 KiB chunks"),
    "gelu_act": Workload(
        "gelu_act", 4096 * 16384, 16384, "qlc", (1, 3, 3, 3, 3, 5, 6, 7), (1,), 16,
        "4096x16384 e4m3 of GELU(N(0,1)); QLC areas (1,3,3,3,3,5,6,7) ranked by a "
        "seed-1 batch; 16 KiB chunks"),
    "int8_weight": Workload(
        "int8_weight", 11008 * 4096, 65536, "huffman", None, (1,), 16,
        "11008x4096 int8 of N(0,0.02), per-row absmax quantized; Huffman-12 from a "
        "seed-1 matrix; 64 KiB chunks"),
    "stream_1g": Workload(
        "stream_1g", 1 << 30, 65536, "huffman", None, (1,), 16,
        "1 GiB e4m3, 16 x 64 MiB segments N(0, sigma_k), sigma_k~U(0.5,2), per-segment "
        "absmax; Huffman-12 from all segments of a seed-1 batch; 64 KiB chunks"),
}

CONFIG_ORDER = ["normal_1m", "ffn1_act", "gelu_act", "int8_weight", "stream_1g"]


def num_segments(name: str) -> int:
    return WORKLOADS[name].segments


def _ffn1_row_scales(seed: int) -> np.ndarray:
    return np.random.default_rng(seed).lognormal(0.0, 0.5, 4096).astype(np.float32)


def _raw_segment_f32(name: str, seed: int, k: int) -> np.ndarray:
    """Float32 values of segment ``k`` before the 8-bit cast."""
    if name == "ffn1_act":
        rows = 4096 // 16
        s = _ffn1_row_scales(seed)[k * rows:(k + 1) * rows]
        x = _seg_rng(seed, k).standard_normal((rows, 16384), dtype=np.float32)
        x *= s[:, None]
        return x.reshape(-1)
    if name == "gelu_act":
        rows = 4096 // 16
        x = _seg_rng(seed, k).standard_normal(rows * 16384, dtype=np.float32)
        return _gelu_erf(x)
    if name == "int8_weight":
        rows = 11008 // 16
        return _seg_rng(seed, k).normal(0.0, 0.02, (rows, 4096)).astype(np.float32)
    if name == "stream_1g":
        sig = np.random.default_rng(seed).uniform(0.5, 2.0, 16).astype(np.float32)
        x = _seg_rng(seed, k).standard_normal(1 << 26, dtype=np.float32)
        x *= sig[k]
        return x
    raise KeyError(name)


def _cast_with_absmax(x: np.ndarray, m: float) -> np.ndarray:
    import torch

    scale = np.float32(E4M3_MAX) / np.float32(m)
    y = x * scale
    np.clip(y, -E4M3_MAX, E4M3_MAX, out=y)
    return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _per_tensor(name: str) -> bool:
    return name in ("ffn1_act", "gelu_act")


def make(name: str, seed: int = 0, threads: int | None = None, out: np.ndarray | None = None) -> np.ndarray:
    """All bytes of workload ``name`` under ``seed`` (uint8, length ``n``)."""
    w = WORKLOADS[name]
    if out is None:
        out = np.empty(w.n, dtype=np.uint8)
    if name == "normal_1m":
        x = np.random.default_rng(seed).standard_normal(w.n, dtype=np.float32)
        out[:] = e4m3_from_f32(x)
        return out
    seg = w.n // w.segments
    threads = threads or min(16, os.cpu_count() or 1)
    pool = _cf.ThreadPoolExecutor(max_workers=threads)
    try:
        if _per_tensor(name):
            # One absmax over the whole tensor: draw every segment first.
            raw = list(pool.map(lambda k: _raw_segment_f32(name, seed, k), range(w.segments)))
            m = max(float(np.abs(r).max()) for r in raw)

            def cast(k):
                out[k * seg:(k + 1) * seg] = _cast_with_absmax(raw[k], m)
                raw[k] = None

            list(pool.map(cast, range(w.segments)))
        else:
            def fill(k):
                x = _raw_segment_f32(name, seed, k)
                if name == "int8_weight":
                    out[k * seg:(k + 1) * seg] = _int8_rows(x)
                else:  # stream_1g: each segment scaled on its own
                    out[k * seg:(k + 1) * seg] = e4m3_from_f32(x)

            list(pool.map(fill, range(w.segments)))
    finally:
        pool.shutdown()
    return out


def make_previous(name: str, seed: int) -> np.ndarray:
    """A previous batch (same recipe, other seed)."""
    return make(name, seed)
