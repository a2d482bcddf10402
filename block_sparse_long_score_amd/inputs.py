"""Seeded synthetic inputs for the MSA hot path.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic.  Both the GPU path (through the tests and the bench)
and the CPU oracle read the same bytes produced here.

Workloads.  The pages measure MSA on long-context evaluation suites at 128K
and on product contexts of 1,048,576 tokens ("MiniMax 模型迭代与竞品分析",
§1 model table and §2 quality table), with M2's attention shape of 48 query
heads and 8 KV heads ("深度解读：The MiniMax-M2 Series", §2).  No suite item is
used: every tensor here is synthetic with those context lengths and head
shapes.

Value recipe (one sub-stream per tensor, seed = 1000 + workload index):
  - Q, K, V: float32 N(0, 1), rounded to nearest-even bfloat16.
  - Q_idx, K_idx: uniform integers in [-4, 4] divided by 4, stored as
    bfloat16.  Every product is a multiple of 1/16 and every partial sum of
    at most 64 such products is exact in float32, so index scores are exact
    in any summation order and block selections can be compared bit for bit.
  - block table: identity for prefill workloads, a seeded random permutation
    of the physical blocks for decode workloads.

Needle variant (workloads with needle_rows > 0).  On i.i.d. inputs the index
keys carry nothing about where the attention mass lies, so selection recall
and coverage sit at chance.  The needle variant plants keys that do: for
each of `needle_rows` evenly spaced query rows r and each KV group g,
`needles_per_group` keys at distinct positions in distinct earlier
(non-local) blocks of r's context get K[i, g] = bf16(gain * Q[r, h]) for one
head h of the group (a different head per needle) and K_idx[i] = Q_idx[r, g]
(an exact copy, so index scores stay exact).  Everything else is the plain
workload's draw.  Positions come from their own seeded sub-stream.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

BLOCK = 128
TOP_K = 16

# Tensor ids of the sub-streams, in a fixed order.
_STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_QIDX, _STREAM_KIDX, _STREAM_TABLE, _STREAM_NEEDLE = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    index_dim: int
    seq_lens: tuple  # tokens per sequence after this step's append
    q_lens: tuple  # query rows per sequence (its last positions)
    permuted_table: bool
    seed: int
    block_size: int = BLOCK
    top_k: int = TOP_K
    needle_rows: int = 0         # query rows that get planted needles (0: plain i.i.d. inputs)
    needles_per_group: int = 4
    needle_gain: float = 1.5

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def total_q(self) -> int:
        return int(sum(self.q_lens))

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return max(math.ceil(n / self.block_size) for n in self.seq_lens)

    def with_sizes(self, name: str, seq_lens, q_lens, permuted_table=None, seed=None, needle_rows=None) -> "Workload":
        """Same head shapes with other sequence sizes (for parity cases)."""
        return dataclasses.replace(
            self, name=name, seq_lens=tuple(int(x) for x in seq_lens), q_lens=tuple(int(x) for x in q_lens),
            permuted_table=self.permuted_table if permuted_table is None else permuted_table,
            seed=self.seed if seed is None else seed,
            needle_rows=self.needle_rows if needle_rows is None else needle_rows)


_M2 = dict(num_q_heads=48, num_kv_heads=8, head_dim=128, index_dim=64)
# M3's attention shape: 64 query heads over 4 KV heads (G = 16), from the
# backbone description in "MiniMax 模型迭代与竞品分析", §3 (native multimodality
# and 1M context).  head_dim and the index dim are not stated; 128 and 64 are
# assumed as for M2.
_M3 = dict(num_q_heads=64, num_kv_heads=4, head_dim=128, index_dim=64)
_ONE_M = 1 << 20

WORKLOADS = {
    "c0": Workload("c0", "tiny MSA prefill, T=4096, 8q/1kv, D=64, d_idx=32",
                   num_q_heads=8, num_kv_heads=1, head_dim=64, index_dim=32,
                   seq_lens=(4096,), q_lens=(4096,), permuted_table=False, seed=1000),
    "c1": Workload("c1", "M2-shaped MSA prefill, T=32768, 48q/8kv, D=128, d_idx=64",
                   seq_lens=(32768,), q_lens=(32768,), permuted_table=False, seed=1001, **_M2),
    "c2": Workload("c2", "MSA decode, 32 sequences x 131072 cached tokens, 48q/8kv",
                   seq_lens=(131072,) * 32, q_lens=(1,) * 32, permuted_table=True, seed=1002, **_M2),
    "c3": Workload("c3", "long MSA prefill, T=131072, 48q/8kv, D=128, d_idx=64",
                   seq_lens=(131072,), q_lens=(131072,), permuted_table=False, seed=1003, **_M2),
    "c4d": Workload("c4d", "1M-context MSA decode, 4 sequences x 1,048,576 cached tokens",
                    seq_lens=(_ONE_M,) * 4, q_lens=(1,) * 4, permuted_table=True, seed=1004, **_M2),
    "c4p": Workload("c4p", "8192-token MSA prefill chunk appended to a 1,048,576-token cache",
                    seq_lens=(_ONE_M + 8192,), q_lens=(8192,), permuted_table=False, seed=1004, **_M2),
    # The 32K prefill and the 32 x 128K decode with planted needles on 64 evenly spaced rows (every
    # decode row): the selection-quality measurements on inputs where the indexer can find the mass.
    "c1n": Workload("c1n", "M2-shaped MSA prefill, T=32768, 48q/8kv, needles planted for 64 rows",
                    seq_lens=(32768,), q_lens=(32768,), permuted_table=False, seed=1001, needle_rows=64, **_M2),
    "c2n": Workload("c2n", "MSA decode, 32 sequences x 131072 cached tokens, 48q/8kv, needles planted for every row",
                    seq_lens=(131072,) * 32, q_lens=(1,) * 32, permuted_table=True, seed=1002, needle_rows=32, **_M2),
    # M3-shaped variants (64q/4kv, G = 16) of the 128K prefill and the 32 x 128K decode.
    "m3p": Workload("m3p", "M3-shaped MSA prefill, T=131072, 64q/4kv (G=16), D=128, d_idx=64",
                    seq_lens=(131072,), q_lens=(131072,), permuted_table=False, seed=1005, **_M3),
    "m3d": Workload("m3d", "M3-shaped MSA decode, 32 sequences x 131072 cached tokens, 64q/4kv (G=16)",
                    seq_lens=(131072,) * 32, q_lens=(1,) * 32, permuted_table=True, seed=1006, **_M3),
}


def _generator(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 16 + stream)
    return g


_CHUNK = 1 << 26  # elements drawn per call, bounds the float32 temporary


def _normal_bf16(shape, gen, device) -> torch.Tensor:
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    for start in range(0, flat.numel(), _CHUNK):
        n = min(_CHUNK, flat.numel() - start)
        flat[start:start + n] = torch.randn(n, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def _dyadic_bf16(shape, gen, device) -> torch.Tensor:
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    for start in range(0, flat.numel(), _CHUNK):
        n = min(_CHUNK, flat.numel() - start)
        ints = torch.randint(-4, 5, (n,), generator=gen, device=device, dtype=torch.int32)
        flat[start:start + n] = ints.to(torch.bfloat16) * 0.25  # exact: a power-of-two scale
    return out


@dataclasses.dataclass
class Inputs:
    """Logical (uncached) tensors of one workload.

    k, v     : bf16 [total_tokens, Hkv, D], sequence s at rows tok_off[s]:tok_off[s+1]
    k_idx    : bf16 [total_tokens, d_idx]
    q        : bf16 [total_q, Hq, D]
    q_idx    : bf16 [total_q, Hkv, d_idx]
    block_table : int32 [num_seqs, max_blocks_per_seq] (physical block ids)
    """
    workload: Workload
    k: torch.Tensor
    v: torch.Tensor
    k_idx: torch.Tensor
    q: torch.Tensor
    q_idx: torch.Tensor
    block_table: torch.Tensor
    num_blocks: int

    @property
    def tok_off(self):
        return np.concatenate([[0], np.cumsum(self.workload.seq_lens)]).astype(np.int64)

    @property
    def cu_q(self):
        return np.concatenate([[0], np.cumsum(self.workload.q_lens)]).astype(np.int32)

    def positions(self, s: int) -> np.ndarray:
        """Absolute positions of sequence s's query rows."""
        n, nq = self.workload.seq_lens[s], self.workload.q_lens[s]
        return np.arange(n - nq, n, dtype=np.int64)

    def new_token_rows(self) -> torch.Tensor:
        """Indices into k/v/k_idx of the tokens this step appends (one per query row)."""
        rows = []
        off = self.tok_off
        for s in range(self.workload.num_seqs):
            n, nq = self.workload.seq_lens[s], self.workload.q_lens[s]
            rows.append(np.arange(off[s] + n - nq, off[s] + n, dtype=np.int64))
        return torch.from_numpy(np.concatenate(rows)).to(self.k.device)


def needle_rows_of(w: Workload) -> np.ndarray:
    """Global query-row indices that carry needles: evenly spaced over all rows."""
    if w.needle_rows <= 0 or w.total_q == 0:
        return np.zeros(0, dtype=np.int64)
    return np.unique(np.linspace(0, w.total_q - 1, min(w.needle_rows, w.total_q)).astype(np.int64))


def needle_plan(w: Workload, seed: int | None = None) -> dict:
    """Where the needles go: int64 arrays row, token (index into k/v/k_idx),
    group, head, one entry per planted key.  Positions are distinct across
    the whole workload, causal for their row and outside its local block."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed * 16 + _STREAM_NEEDLE)
    cu = np.concatenate([[0], np.cumsum(w.q_lens)]).astype(np.int64)
    off = np.concatenate([[0], np.cumsum(w.seq_lens)]).astype(np.int64)
    B, G = w.block_size, w.group_size
    used = set()
    out = {"row": [], "token": [], "group": [], "head": []}
    for r in needle_rows_of(w):
        s = int(np.searchsorted(cu, r, side="right") - 1)
        t = w.seq_lens[s] - int(cu[s + 1] - r)
        c = t // B
        if c == 0:
            continue
        for g in range(w.num_kv_heads):
            blocks = rng.choice(c, size=min(w.needles_per_group, c), replace=False)
            for n, b in enumerate(blocks):
                for _ in range(8):
                    tok = int(off[s] + b * B + rng.integers(0, B))
                    if tok not in used:
                        used.add(tok)
                        out["row"].append(int(r))
                        out["token"].append(tok)
                        out["group"].append(g)
                        out["head"].append(g * G + n % G)
                        break
    return {k: np.asarray(v, dtype=np.int64) for k, v in out.items()}


def make_inputs(w: Workload, device="cpu", seed: int | None = None) -> Inputs:
    """Draw every tensor of workload `w` on `device` from its seeded sub-streams."""
    seed = w.seed if seed is None else seed
    dev = torch.device(device)
    hkv, d, di = w.num_kv_heads, w.head_dim, w.index_dim
    q = _normal_bf16((w.total_q, w.num_q_heads, d), _generator(dev, seed, _STREAM_Q), dev)
    k = _normal_bf16((w.total_tokens, hkv, d), _generator(dev, seed, _STREAM_K), dev)
    v = _normal_bf16((w.total_tokens, hkv, d), _generator(dev, seed, _STREAM_V), dev)
    q_idx = _dyadic_bf16((w.total_q, hkv, di), _generator(dev, seed, _STREAM_QIDX), dev)
    k_idx = _dyadic_bf16((w.total_tokens, di), _generator(dev, seed, _STREAM_KIDX), dev)
    mb = w.max_blocks_per_seq
    num_blocks = w.num_seqs * mb
    if w.permuted_table:
        perm = torch.randperm(num_blocks, generator=_generator(dev, seed, _STREAM_TABLE), device=dev)
        table = perm.to(torch.int32).view(w.num_seqs, mb)
    else:
        table = torch.arange(num_blocks, device=dev, dtype=torch.int32).view(w.num_seqs, mb)
    if w.needle_rows > 0:
        plan = {key: torch.from_numpy(val).to(dev) for key, val in needle_plan(w, seed).items()}
        if plan["token"].numel():
            k[plan["token"], plan["group"]] = (q[plan["row"], plan["head"]].float() * w.needle_gain).to(torch.bfloat16)
            k_idx[plan["token"]] = q_idx[plan["row"], plan["group"]]
    return Inputs(w, k, v, k_idx, q, q_idx, table.contiguous(), num_blocks)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy, no arithmetic)."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bfloat16 tensor")
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
