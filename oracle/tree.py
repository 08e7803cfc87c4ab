"""The fixed fp32 reduction tree, replayed one IEEE operation at a time.

Source: "Defeating nondeterminism in LLM inference", section on batch-invariant
RMSNorm: the order in which each row is reduced must be fixed whatever the batch
size; it may depend on the reduced length, and the reduction may go thread ->
warp -> block.  The tree below is a function of the row length n and the vector
width w only (never of the number of rows):

  T = min(256, ceil(n / w)) lanes, grouped in waves of 64 lanes.
  Vector v holds elements [w*v, w*v + w); lane t owns vectors t, t+T, t+2T, ...
  1. each lane adds its elements in ascending index order into an fp32
     accumulator that starts at +0;
  2. inside each wave: butterfly exchange with lane offsets 1, 2, 4, 8, 16, 32 in
     that order (because fp32 addition is commutative this is the index-order
     pairwise tree over the 64 lanes; lanes that own nothing hold +0);
  3. across waves: index-order pairwise tree, a missing fourth wave counts as +0
     ((w0 + w1) + (w2 + w3)).
"""
from __future__ import annotations

import numpy as np

MAX_LANES = 256
WAVE = 64


def lanes_for(n: int, width: int) -> int:
    return max(1, min(MAX_LANES, -(-n // width)))


def lane_partials(vals: np.ndarray, width: int) -> np.ndarray:
    """Step 1 for every row at once: vals [M, n] float32 -> acc [M, T] float32."""
    vals = np.asarray(vals, dtype=np.float32)
    m, n = vals.shape
    t = lanes_for(n, width)
    nvec = -(-n // width)
    steps = -(-nvec // t)
    acc = np.zeros((m, t), dtype=np.float32)
    idx_lane = np.arange(t)
    for s in range(steps):
        for e in range(width):
            idx = (s * t + idx_lane) * width + e          # element index owned by each lane
            valid = idx < n
            col = vals[:, np.minimum(idx, n - 1)]
            acc = np.where(valid[None, :], acc + col, acc)
    return acc


def combine_lanes(acc: np.ndarray) -> np.ndarray:
    """Steps 2 and 3: acc [M, T] -> [M]."""
    m, t = acc.shape
    n_waves = -(-t // WAVE)
    full = np.zeros((m, n_waves * WAVE), dtype=np.float32)
    full[:, :t] = acc
    waves = full.reshape(m, n_waves, WAVE)
    for _ in range(6):                                    # offsets 1, 2, 4, 8, 16, 32
        waves = waves[:, :, 0::2] + waves[:, :, 1::2]
    w = waves[:, :, 0]                                    # [M, n_waves]
    if n_waves == 1:
        return w[:, 0]
    if n_waves == 2:
        return w[:, 0] + w[:, 1]
    pad = np.zeros((m, 4), dtype=np.float32)
    pad[:, :n_waves] = w
    return (pad[:, 0] + pad[:, 1]) + (pad[:, 2] + pad[:, 3])


def tree_sum(vals: np.ndarray, width: int) -> np.ndarray:
    return combine_lanes(lane_partials(vals, width))


def sequential_sum(vals: np.ndarray) -> np.ndarray:
    """Left-to-right fp32 sum (used only to show that the order matters)."""
    vals = np.asarray(vals, dtype=np.float32)
    acc = np.zeros(vals.shape[0], dtype=np.float32)
    for j in range(vals.shape[1]):
        acc = acc + vals[:, j]
    return acc
