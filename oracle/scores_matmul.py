"""Steps 1-2 of MSA (index scores, 128-token block max-pool) for many query
rows at once, as a matrix product — TEST INFRASTRUCTURE, like the rest of
``oracle/``.

"MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2, steps 1-2: every
query row t scores each causal key i <= t by the dot product of its group's
Q_idx with the shared K_idx[i]; the scores of each 128-token block are
reduced by max (the local block over its causal part only).

For all scores of a set of rows against all keys this is one matrix product
S = Q_idx K_idx^T per group, which a library matmul computes.  It is exact
(equal to the correctly rounded dot product of ``msa_oracle.c``, and to the
exact value) only when every partial sum is representable in float32 in any
order: this module checks that the inputs are dyadic, i.e. multiples of 2^-e
whose products and sums stay within float32's 24-bit significand, and
refuses other inputs.  The workloads' index inputs (integers in [-4, 4]
divided by 4) satisfy it with a wide margin.  It serves where the C loop
would take minutes (every row of a 131,072-token prefill); it is pinned bit
for bit to ``msa_oracle_block_scores`` on the CPU.
"""
from __future__ import annotations

import numpy as np
import torch


def _bits_to_f32(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy((a.astype(np.uint32) << 16).view(np.float32))


def _dyadic_exponent(x: torch.Tensor) -> int:
    """Smallest e >= 0 with x * 2^e integral everywhere (ValueError if none up to 2^20)."""
    for e in range(21):
        y = x * float(1 << e)
        if bool(torch.all(y == torch.round(y))):
            return e
    raise ValueError("index inputs are not dyadic: the float32 matrix product would not be exact")


def block_scores(first_pos: int, q_idx: np.ndarray, k_idx: np.ndarray, block_size: int = 128,
                 ld: int | None = None, rows_per_batch: int = 512) -> np.ndarray:
    """Pooled index scores of consecutive query rows at positions
    first_pos, first_pos + 1, ... (one sequence).

    q_idx : uint16 [n, G, d_idx] bf16 bits; k_idx : uint16 [L, d_idx] bf16 bits, L > last position.
    returns float32 [n, G, ld]; entries after each row's own block are -inf.
    """
    q = _bits_to_f32(q_idx)
    k = _bits_to_f32(k_idx)
    n, groups, d = q.shape
    last = first_pos + n - 1
    if n == 0:
        return np.zeros((0, groups, ld or 1), np.float32)
    if k.shape[0] <= last:
        raise ValueError("k_idx must hold every key up to the last query position")
    if ld is None:
        ld = last // block_size + 1
    # Exactness: with x = a 2^-eq and y = b 2^-ek (a, b integers), every partial sum of a
    # d-term dot product is an integer multiple of 2^-(eq+ek) bounded by d max|a| max|b|.
    eq, ek = _dyadic_exponent(q), _dyadic_exponent(k)
    bound = d * float(q.abs().max()) * (1 << eq) * float(k.abs().max()) * (1 << ek)
    if bound >= 2.0 ** 24:
        raise ValueError("index inputs too wide for an exact float32 product")
    out = np.full((n, groups, ld), -np.inf, np.float32)
    for r0 in range(0, n, rows_per_batch):
        r1 = min(n, r0 + rows_per_batch)
        t = torch.arange(first_pos + r0, first_pos + r1)                   # positions of the rows
        nkeys = int(t[-1]) + 1
        # Blocks below the batch's first row are causal for every row of the batch; the
        # blocks from there on hold keys after some rows, which the causal mask removes.
        nfull = (first_pos + r0) // block_size
        ntail = (nkeys + block_size - 1) // block_size - nfull
        tail_keys = torch.arange(nfull * block_size, (nfull + ntail) * block_size)
        causal = tail_keys[None, :] <= t[:, None]                          # step 1: keys i <= t only
        tail = torch.zeros((ntail * block_size, d), dtype=torch.float32)
        tail[: nkeys - nfull * block_size] = k[nfull * block_size: nkeys]
        for g in range(groups):
            qg = q[r0:r1, g]
            if nfull:
                s = qg @ k[: nfull * block_size].T                         # step 1: dot products
                pooled = s.view(r1 - r0, nfull, block_size).amax(dim=2)    # step 2: max per block
                out[r0:r1, g, :nfull] = (pooled + 0.0).numpy()             # -0 and +0 are one score
            s = torch.where(causal, qg @ tail.T, torch.tensor(-np.inf))
            pooled = s.view(r1 - r0, ntail, block_size).amax(dim=2)
            out[r0:r1, g, nfull:nfull + ntail] = (pooled + 0.0).numpy()
    return out
