"""Independent textbook references used to pin the oracle (numpy, float64).

Nothing here is shared with the oracle: these are the plain definitions the
MSA oracle must reduce to in special cases.
  - dense_causal_gqa: softmax attention of the equation in "MiniMax
    模型迭代与竞品分析" §2 (scores q.k/sqrt(d), softmax over all keys j <= t,
    probability-weighted sum of values), with GQA head sharing.
  - full_score_matrix / pool_by_loops: the whole T x T index-score matrix
    and its block max-pool written as explicit loops.
  - dominance_selection: top-k defined by dominance (every kept block beats
    every dropped block in the order score-descending, index-ascending), found
    by enumerating every subset.
"""
import itertools

import numpy as np


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def dense_causal_gqa(q, k, v, pos, scale):
    """q [n,Hq,D], k/v [L,G,D] float64; out [n,Hq,D]."""
    n, hq, _ = q.shape
    groups = k.shape[1]
    gs = hq // groups
    out = np.empty_like(q)
    for r in range(n):
        t = int(pos[r])
        for h in range(hq):
            g = h // gs
            z = scale * (k[: t + 1, g, :] @ q[r, h])
            p = np.exp(z - z.max())
            p /= p.sum()
            out[r, h] = p @ v[: t + 1, g, :]
    return out


def full_score_matrix(q_idx, k_idx):
    """q_idx [n,G,di], k_idx [L,di] (float64) -> scores [n,G,L]."""
    return np.einsum("ngd,ld->ngl", q_idx, k_idx)


def pool_by_loops(scores, pos, block_size, ld):
    n, groups, _ = scores.shape
    pooled = np.full((n, groups, ld), -np.inf)
    for r in range(n):
        for g in range(groups):
            for i in range(int(pos[r]) + 1):
                b = i // block_size
                pooled[r, g, b] = max(pooled[r, g, b], scores[r, g, i])
    return pooled


def dominance_selection(pooled_row, c, top_k):
    """The unique set: local block c plus top_k-1 of blocks < c such that every
    kept block beats every dropped one (higher score, or equal score and lower
    index).  Found by trying every subset.  Returns the ascending list."""
    if c + 1 <= top_k:
        return list(range(c + 1))

    def beats(a, b):
        return pooled_row[a] > pooled_row[b] or (pooled_row[a] == pooled_row[b] and a < b)

    found = []
    for subset in itertools.combinations(range(c), top_k - 1):
        kept = set(subset)
        if all(beats(a, b) for a in kept for b in range(c) if b not in kept):
            found.append(sorted(kept) + [c])
    assert len(found) == 1, f"dominance must single out one subset, found {len(found)}"
    return found[0]
