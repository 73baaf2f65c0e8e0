"""Codebook refresh: a fixed codebook from the pooled histograms of recent
batches, rebuilt when it stops fitting the data.

"Single-Stage Huffman Encoder for ML Compression" (abstract) builds the one
codebook from the average distribution of previous batches; the Shannonic
page ("Shannonic: Efficient Entropy-Optimal Compression for ML Workloads",
key observation 1) expects static tables to be refreshed when the
distribution drifts.  This is the host-side policy around the library:
histograms come from ``pc_histogram`` (device; ``observe_batch`` also pools
them there), the fit test from ``pc_codebook_fit`` and the build from
``pc_codebook_build`` (host C).
"""
from __future__ import annotations

from collections import deque

import numpy as np
import torch

from ._lib import pc_codebook_build, pc_codebook_fit, pc_histogram, pc_qlc_optimal_bits

__all__ = ["CodebookRefresh"]


class CodebookRefresh:
    """Keeps the byte histograms of the last ``window`` batches.

    ``observe(counts)`` first measures how the current codebook fits the new
    batch (bits per symbol against the batch's entropy), then adds the batch
    to the pool.  When there is no codebook yet, or the relative gap
    ``(avg_bits - entropy) / entropy`` exceeds ``threshold``, the codebook is
    rebuilt from the pooled counts (summing the histograms of equal-size
    batches is proportional to averaging their distributions) and
    ``observe`` returns True.  For QLC codebooks with ``qlc_bits=None`` the
    area widths are chosen for the pooled counts by ``pc_qlc_optimal_bits``.
    """

    def __init__(self, kind: str = "huffman", qlc_bits=None, window: int = 8, threshold: float = 0.02):
        if window < 1:
            raise ValueError("window must be >= 1")
        if threshold < 0:
            raise ValueError("threshold must be >= 0")
        self.kind, self.qlc_bits, self.threshold = kind, qlc_bits, float(threshold)
        self.window = window
        self.pool: deque = deque(maxlen=window)
        self.codebook: torch.Tensor | None = None  # host blob (CPU uint8)
        self.last_fit: tuple | None = None         # (avg_bits, entropy) of the last batch
        self.rebuilds = 0
        # device pool (observe_batch): the pooled histogram accumulated by
        # pc_histogram, and each pooled batch's own histogram, to take it out
        # again when it leaves the window
        self.pool_dev: torch.Tensor | None = None
        self.ring_dev: deque = deque()

    def pooled(self) -> np.ndarray:
        return np.sum(np.stack(list(self.pool)), axis=0).astype(np.uint64)

    def gap(self, counts) -> float:
        """Relative excess of the current codebook over the batch's entropy."""
        avg, ent = pc_codebook_fit(self.codebook, counts)
        self.last_fit = (avg, ent)
        return (avg - ent) / ent if ent > 0 else 0.0

    def observe_batch(self, d_batch: torch.Tensor) -> bool:
        """``observe`` for a batch of bytes on the device: ``pc_histogram``
        counts the batch into its own histogram and adds it to the pooled
        one, both on the device (the pool is the sum over the last
        ``window`` batches; a batch leaving the window is subtracted again).
        Only the 256 counts cross to the host, for the fit test and the
        build.  Do not mix with ``observe`` on one object."""
        dev = d_batch.device
        if self.pool_dev is None:
            self.pool_dev = torch.zeros(256, dtype=torch.int64, device=dev)
        h = pc_histogram(d_batch)
        pc_histogram(d_batch, self.pool_dev)
        self.ring_dev.append(h)
        if len(self.ring_dev) > self.window:
            self.pool_dev.sub_(self.ring_dev.popleft())
        c = h.cpu().numpy().astype(np.uint64)
        stale = self.codebook is None or self.gap(c) > self.threshold
        if not stale:
            return False
        self._rebuild(self.pool_dev.cpu().numpy().astype(np.uint64))
        return True

    def _rebuild(self, pooled: np.ndarray) -> None:
        bits = self.qlc_bits
        if self.kind == "qlc" and bits is None:
            bits = pc_qlc_optimal_bits(pooled)
        self.codebook = pc_codebook_build(pooled, self.kind, bits if self.kind == "qlc" else None)
        self.rebuilds += 1

    def observe(self, counts) -> bool:
        c = np.asarray(counts.cpu() if isinstance(counts, torch.Tensor) else counts).astype(np.uint64)
        if c.shape != (256,):
            raise ValueError("counts must have 256 entries")
        stale = self.codebook is None or self.gap(c) > self.threshold
        self.pool.append(c)
        if not stale:
            return False
        self._rebuild(self.pooled())
        return True
