"""The seeded input generator (CPU): the needle variant plants exactly what
its recipe says and leaves every other value of the plain draw unchanged."""
import numpy as np
import torch

from block_sparse_long_score_amd.inputs import WORKLOADS, make_inputs, needle_plan, needle_rows_of


def _small(needle_rows, **kw):
    return WORKLOADS["c1n"].with_sizes("needle_small", [3000, 700], [2000, 700], needle_rows=needle_rows, **kw)


def test_needles_are_planted_as_described():
    w = _small(12)
    inp = make_inputs(w, "cpu")
    plan = needle_plan(w)
    assert len(plan["token"]) > 0
    assert len(set(plan["token"].tolist())) == len(plan["token"]), "needle positions must be distinct"
    cu = inp.cu_q
    off = inp.tok_off
    gain = torch.tensor(w.needle_gain, dtype=torch.float32)
    for r, tok, g, h in zip(plan["row"], plan["token"], plan["group"], plan["head"]):
        s = int(np.searchsorted(cu, r, side="right") - 1)
        t = w.seq_lens[s] - int(cu[s + 1] - r)
        i = int(tok - off[s])
        assert 0 <= i < (t // 128) * 128, "needle must be causal and outside the row's local block"
        assert g * w.group_size <= h < (g + 1) * w.group_size, "needle head must belong to its group"
        assert torch.equal(inp.k_idx[tok], inp.q_idx[r, g])
        assert torch.equal(inp.k[tok, g], (inp.q[r, h].float() * gain).to(torch.bfloat16))
    # at most needles_per_group per (row, group), in distinct blocks of the row's sequence
    for r in np.unique(plan["row"]):
        s = int(np.searchsorted(cu, r, side="right") - 1)
        for g in range(w.num_kv_heads):
            sel = (plan["row"] == r) & (plan["group"] == g)
            assert sel.sum() <= w.needles_per_group
            assert len(np.unique((plan["token"][sel] - off[s]) // 128)) == sel.sum()


def test_needles_leave_the_rest_of_the_draw_unchanged():
    w = _small(12)
    plain = make_inputs(w.with_sizes("plain", w.seq_lens, w.q_lens, needle_rows=0), "cpu")
    inp = make_inputs(w, "cpu")
    touched = torch.zeros(w.total_tokens, dtype=torch.bool)
    touched[torch.from_numpy(needle_plan(w)["token"])] = True
    assert torch.equal(inp.q, plain.q) and torch.equal(inp.q_idx, plain.q_idx) and torch.equal(inp.v, plain.v)
    assert torch.equal(inp.k_idx[~touched], plain.k_idx[~touched])
    assert torch.equal(inp.k[~touched], plain.k[~touched])
    # within a touched token only the needle's own group changes
    plan = needle_plan(w)
    for tok, g in zip(plan["token"], plan["group"]):
        others = [x for x in range(w.num_kv_heads) if x != g and not ((plan["token"] == tok) & (plan["group"] == x)).any()]
        assert torch.equal(inp.k[tok, others], plain.k[tok, others])


def test_needle_rows_are_evenly_spaced_and_seeded():
    w = _small(12)
    rows = needle_rows_of(w)
    assert len(rows) == 12 and rows[0] == 0 and rows[-1] == w.total_q - 1
    a, b = needle_plan(w), needle_plan(w)
    assert all(np.array_equal(a[k], b[k]) for k in a)
    c = needle_plan(w, seed=w.seed + 1)
    assert not np.array_equal(a["token"], c["token"])
    assert len(needle_rows_of(_small(0))) == 0
