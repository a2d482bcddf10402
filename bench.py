"""Throughput of the MSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

A step is one pass of the whole hot path over one batch of synthetic input,
through the C ABI: append the batch's new K/V/K_idx to the block-major cache,
index scoring + block max-pool, top-16 block selection, and the Main Branch
(prefill: every query row of the chunk; decode: one new token per sequence).
Inputs are resident in HBM before timing starts.  Prints one JSON line.

The default workload is the 131,072-token prefill (48 query heads / 8 KV
heads, head_dim 128, index dim 64), the context length the metric is quoted
at; --workload selects another (c0 tiny prefill, c1 32K prefill, c2 decode of
32 x 128K, c4d decode of 4 x 1M, c4p 8K chunk onto a 1M cache, m3p / m3d the
same 128K prefill and 32 x 128K decode with M3's 64 query / 4 KV heads, c1n / c2n
c1 / c2 with needles planted for the rows whose selection quality is measured).
With the default c3 headline, the same run then measures c1 and the 8K
chunk onto a 1M cache (prefill) and the 32 x 128K and 4 x 1M decodes, each
reported under "legs" with its tokens/s, whole-step fraction of peak and the
roofline of its dominant stage (--legs selects others, or none).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "MSA prefill tokens/s & decode tokens/s at 128K/1M ctx; % MFMA / % HBM peak"


def algorithmic_work(w):
    """Per-step algorithmic flops and bytes of each stage (what the method
    must compute/move, independent of how the kernels do it)."""
    B = w.block_size
    idx_flops = main_flops = 0.0
    kidx_bytes = kv_bytes = 0.0
    for n, nq in zip(w.seq_lens, w.q_lens):
        t = np.arange(n - nq, n, dtype=np.float64)
        c = np.floor(t / B)
        # attended tokens: every causal token below 16 blocks, else 15 full blocks + the causal part of the local one
        lsel = np.where(c + 1 <= w.top_k, t + 1, (w.top_k - 1) * B + (t - c * B + 1))
        idx_flops += 2.0 * w.index_dim * w.num_kv_heads * float(np.sum(t + 1))
        main_flops += 4.0 * w.head_dim * w.num_q_heads * float(np.sum(lsel))
        kidx_bytes += 2.0 * w.index_dim * float(np.sum(t + 1)) if nq == 1 else 2.0 * w.index_dim * n
        kv_bytes += 2.0 * 2.0 * w.head_dim * w.num_kv_heads * float(np.sum(lsel))
    nblk = sum((n + B - 1) // B for n in w.seq_lens)
    rows = w.total_q
    io_bytes = (rows * w.num_q_heads * w.head_dim * 2 * 2            # q in, out
                + rows * w.num_kv_heads * w.index_dim * 2            # q_idx
                + rows * (2 * w.num_kv_heads * w.head_dim + w.index_dim) * 2 * 2  # append: read + write
                + rows * w.num_kv_heads * w.top_k * 4)               # selections
    pooled_bytes = 2 * 4 * w.num_kv_heads * sum(nq * (n + B - 1) // B for n, nq in zip(w.seq_lens, w.q_lens))
    return dict(index_flops=idx_flops, main_flops=main_flops, kidx_bytes=kidx_bytes, kv_bytes=kv_bytes,
                io_bytes=float(io_bytes), pooled_bytes=float(pooled_bytes), nblk=nblk)


def _code_only(text: str) -> str:
    """C++ source without its comments and blank space, so that a comment edit
    leaves the hash of the code (and the profiles recorded for it) valid.
    String and character literals are kept as they are."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the code (comments and spacing aside) of the HIP sources and
    headers the library is built from."""
    import hashlib
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "block_sparse_long_score_amd", "csrc"), os.path.join(ROOT, "include")):
        for f in sorted(os.listdir(d)):
            if f.endswith((".hip", ".h")):
                h.update(f.encode())
                with open(os.path.join(d, f), encoding="utf-8") as fh:
                    h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, stage: str, launches_per_step: float):
    """HBM bytes per launch of a stage, from the rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs recorded under profiles/ (scaled by the copy-kernel calibration
    recorded with them); None if none was recorded for this workload or the
    kernels changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload, {}).get(stage)
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return {"bytes_per_launch": rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"],
            "read_bytes_per_launch": rec["read_bytes_per_launch"], "write_bytes_per_launch": rec["write_bytes_per_launch"],
            "source": rec["profile"]}


def selection_quality(runner, n_rows: int):
    """Coverage and recall of the step's selections on evenly spaced query rows
    against the dense attention mass (msa_block_attn_mass), and the indexer's
    D_KL(P||Q) over each row's candidate blocks, P the Main Branch's mass over
    them (msa_block_attn_mass with the selections), with the dense mass kernel
    timed by events.  After the timed region; not part of a step."""
    import torch
    from block_sparse_long_score_amd import ops
    w, dev = runner.inputs.workload, runner.inputs.q.device
    n = min(n_rows, w.total_q)
    rows = torch.from_numpy(np.unique(np.linspace(0, w.total_q - 1, n).astype(np.int32))).to(dev)
    mass = torch.empty((rows.numel(), w.num_kv_heads, runner.ld), dtype=torch.float32, device=dev)
    sel_mass = torch.empty_like(mass)
    qual = torch.empty((rows.numel(), w.num_kv_heads, 3), dtype=torch.float32, device=dev)
    runner.step()  # the selections and scores of one step
    ops.msa_block_attn_mass(runner.dims, runner.cache, runner.batch, runner.inputs.q, rows, mass)  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    ops.msa_block_attn_mass(runner.dims, runner.cache, runner.batch, runner.inputs.q, rows, mass)
    e1.record()
    ops.msa_block_attn_mass(runner.dims, runner.cache, runner.batch, runner.inputs.q, rows, sel_mass, sel=runner.sel)
    ops.msa_selection_quality(runner.dims, runner.batch, rows, mass, sel_mass, runner.scores, runner.sel, qual)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    # positions of the sampled rows -> keys each (row, group) scans: t + 1 (read twice by the two passes)
    cu = np.asarray(runner.inputs.cu_q)
    r = rows.cpu().numpy()
    seq = np.searchsorted(cu, r, side="right") - 1
    pos = np.asarray(w.seq_lens)[seq] - (cu[seq + 1] - r)
    k_bytes = float(np.sum(pos + 1)) * w.num_kv_heads * w.head_dim * 2
    q = qual.cpu().numpy().astype(np.float64)
    blocks = pos // w.block_size + 1
    return {"rows": int(rows.numel()), "coverage_mean": float(q[..., 0].mean()), "recall_mean": float(q[..., 1].mean()),
            "kl_candidates_mean": float(q[..., 2].mean()),
            "uniform_coverage_mean": float(np.mean(np.minimum(w.top_k, blocks) / blocks)),
            "mass_kernel_ms": ms, "mass_kernel_gbs": 2 * k_bytes / (ms / 1e3) / 1e9}


def dense_attention(runner, n_calls: int):
    """The dense path on the same batch and cache (msa_dense_attn_prefill or,
    for decode, msa_dense_attn_decode: every causal key attended), timed by
    events over n_calls calls after the timed region; not part of a step.
    Gives an in-repo dense attention time to set beside the sparse Main
    Branch and the whole MSA step."""
    import torch
    from block_sparse_long_score_amd import ops
    w = runner.inputs.workload
    out = torch.empty_like(runner.inputs.q)
    if runner.decode:
        need = ops.msa_workspace_size(runner.dims, runner.cache, runner.batch, ops.MSA_CALL_DENSE_ATTN_DECODE)
        ws = torch.empty(need, dtype=torch.uint8, device=out.device)
        call = lambda: ops.msa_dense_attn_decode(runner.dims, runner.cache, runner.batch, runner.inputs.q, out, ws)
    else:
        call = lambda: ops.msa_dense_attn_prefill(runner.dims, runner.cache, runner.batch, runner.inputs.q, out)
    call()  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_calls):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_calls
    flops = 0.0
    for n, nq in zip(w.seq_lens, w.q_lens):
        t = np.arange(n - nq, n, dtype=np.float64)
        flops += 4.0 * w.head_dim * w.num_q_heads * float(np.sum(t + 1))
    if runner.decode:  # HBM-bound: every cached K and V row read once per (sequence, group)
        kv = sum(2.0 * 2 * w.head_dim * w.num_kv_heads * n for n in w.seq_lens)
        gbs = kv / (ms / 1e3) / 1e9
        return {"kernel": "msa_dense_attn_decode (dense_decode_kernel + dense_decode_merge_kernel)", "calls": n_calls,
                "ms": ms, "algorithmic_bytes": kv, "achieved_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                "traffic": recorded_traffic(w.name, "dense", 1.0)}
    tflops = flops / (ms / 1e3) / 1e12
    return {"kernel": "msa_dense_attn_prefill (dense_prefill_kernel)", "calls": n_calls, "ms": ms,
            "algorithmic_flops": flops, "achieved_tflops": tflops, "mfma_frac": tflops / BF16_PEAK_TFLOPS,
            "traffic": recorded_traffic(w.name, "dense", 1.0)}


def cpu_baseline(inputs, runner, budget_s: float):
    """The oracle as it stands, on a bounded sample of the same workload's
    rows, timed on this host's cores.  Host copies are outside the timing."""
    import oracle
    from block_sparse_long_score_amd.inputs import bf16_bits
    import torch

    w = inputs.workload
    B = w.block_size

    def run_rows(s, positions):
        rows = torch.from_numpy(inputs.cu_q[s] + positions - (w.seq_lens[s] - w.q_lens[s])).to(inputs.q.device)
        off = int(inputs.tok_off[s])
        length = int(positions.max()) + 1
        k_idx = bf16_bits(inputs.k_idx[off:off + length])
        q_idx = bf16_bits(inputs.q_idx.index_select(0, rows))
        q = bf16_bits(inputs.q.index_select(0, rows))
        t0 = time.perf_counter()
        pooled = oracle.block_scores(positions, q_idx, k_idx, B, (w.seq_lens[s] + B - 1) // B)
        sel = oracle.select(positions, pooled, B, w.top_k)
        t_sel = time.perf_counter() - t0
        blocks = np.unique(sel[sel >= 0]).astype(np.int64)
        tok = (blocks[:, None] * B + np.arange(B)[None, :]).ravel()
        tok = tok[tok < length]
        shape = (length, w.num_kv_heads, w.head_dim)
        k_host = np.zeros(shape, np.uint16)
        v_host = np.zeros(shape, np.uint16)
        tok_dev = torch.from_numpy(tok + off).to(inputs.k.device)
        k_host[tok] = bf16_bits(inputs.k.index_select(0, tok_dev))
        v_host[tok] = bf16_bits(inputs.v.index_select(0, tok_dev))
        t0 = time.perf_counter()
        oracle.attend(positions, q, k_host, v_host, sel, B)
        return t_sel + time.perf_counter() - t0

    decode = runner.decode
    all_threads = oracle.num_threads()
    if decode:
        # whole decode rows (one per sequence), sequences taken in order until the budget is spent
        spent, n = 0.0, 0
        for s in range(w.num_seqs):
            spent += run_rows(s, np.array([w.seq_lens[s] - 1], np.int64))
            n += 1
            if spent >= budget_s:
                break
        # one row per call: the scoring loop runs over that row's groups, its attention on one thread
        used = min(all_threads, w.num_kv_heads)
        sample = (f"{n} of {w.num_seqs} decode rows (full {w.seq_lens[0]}-token context each), one row per call: "
                  f"scoring spread over the row's {w.num_kv_heads} groups, attention on one thread")
        value = n / spent
        oracle.set_num_threads(1)
        one = 1.0 / run_rows(0, np.array([w.seq_lens[0] - 1], np.int64))
        sample1 = "1 decode row"
    else:
        s = 0
        n_q = w.q_lens[0]
        first = w.seq_lens[0] - n_q
        # grow the evenly spaced sample until it holds about `budget_s` of oracle work
        n = 16
        while True:
            pos = np.unique(np.linspace(first, w.seq_lens[0] - 1, n).astype(np.int64))
            spent = run_rows(s, pos)
            if spent >= budget_s / 2 or n >= n_q:
                break
            n = int(min(n_q, max(2 * n, n * budget_s / max(spent, 1e-3))))
        sample = f"{len(pos)} query rows evenly spaced over positions {first}..{w.seq_lens[0] - 1} (all groups/heads)"
        value = len(pos) / spent
        used = all_threads
        pos1 = pos[:: max(1, len(pos) // max(4, len(pos) // (2 * all_threads)))]
        oracle.set_num_threads(1)
        one = len(pos1) / run_rows(s, pos1)
        sample1 = f"every {max(1, len(pos) // max(4, len(pos) // (2 * all_threads)))}th row of that sample ({len(pos1)} rows)"
    oracle.set_num_threads(all_threads)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": value, "unit": "tokens/s", "cores": used, "kind": "oracle", "sample": sample,
            "seconds": round(spent, 2), "value_1_thread": one, "sample_1_thread": sample1, "host_cpu": cpu,
            "host_logical_cpus": os.cpu_count()}


def workload_leg(name: str, steps: int, warmup: int, chunk_rows: int):
    """One more workload measured in the same run, after the headline one: its
    steps timed back to back (decode steps rotating over two cache copies),
    each launch of its dominant stage bracketed by events on its stream for
    the roofline, and a serial stage breakdown.  Its buffers are freed before
    returning."""
    import torch
    from block_sparse_long_score_amd.inputs import WORKLOADS, make_inputs
    from block_sparse_long_score_amd.pipeline import MsaRunner

    w = WORKLOADS[name]
    inputs = make_inputs(w, "cuda")
    runner = MsaRunner(inputs, chunk_rows=chunk_rows or None)
    runners = [runner] + ([MsaRunner(inputs)] if runner.decode else [])
    n_rot = len(runners)
    stream = torch.cuda.current_stream()
    for i in range(warmup * n_rot):
        runners[i % n_rot].step()
    torch.cuda.synchronize()

    def serial_stages():
        out, marks = {}, []

        def mark(stage):
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            marks.append((stage, e))

        runner.staged_step(mark)
        torch.cuda.synchronize()
        for (_, e0), (stage, e1) in zip(marks, marks[1:]):
            out[stage] = out.get(stage, 0.0) + e0.elapsed_time(e1)
        return out

    stage_ms = serial_stages()
    dom = "index_score" if runner.decode else max(("index_score", "attend"), key=lambda k: stage_ms[k])
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        runners[i % n_rot].step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    pairs = []

    def hook(stage, st, phase):
        if stage != dom:
            return
        e = torch.cuda.Event(enable_timing=True)
        e.record(st)
        if phase == 0:
            pairs.append([e, None])
        else:
            pairs[-1][1] = e

    for r in runners:
        r.hook = hook
    for i in range(steps):
        runners[i % n_rot].step(fused=False)  # the four calls one by one, so the stage can be bracketed
    torch.cuda.synchronize()
    for r in runners:
        r.hook = None
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in pairs]))
    launches = len(pairs) / steps
    work = algorithmic_work(w)
    leg = {"workload": f"{w.name}: {w.description}", "mode": "decode" if runner.decode else "prefill",
           "steps": steps, "warmup": warmup, "ms_per_step": ms, "tokens_per_s": w.total_q / (ms / 1e3),
           "stage_ms_serial": stage_ms,
           "step_calls": "msa_decode_step" if runner.decode else "msa_kv_append + msa_index_score + msa_block_topk + "
                                                                 "msa_sparse_attn_prefill per chunk"}
    if runner.decode:
        algo = (work["kidx_bytes"] + work["pooled_bytes"] / 2) / launches
        gbs = algo / (launch_ms / 1e3) / 1e9
        step_bytes = work["kidx_bytes"] + work["kv_bytes"] + work["io_bytes"] + work["pooled_bytes"]
        leg["cache_copies_rotated"] = n_rot
        leg["hbm_frac_whole_step"] = step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS
        leg["algorithmic_bytes_per_step"] = step_bytes
        leg["roofline"] = {"bound": "hbm", "stage": dom, "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": gbs / HBM_PEAK_GBS, "avg_launch_ms": launch_ms,
                           "algorithmic_bytes_per_launch": algo, "traffic": recorded_traffic(w.name, dom, launches)}
    else:
        algo = (work["index_flops"] if dom == "index_score" else work["main_flops"]) / launches
        tf = algo / (launch_ms / 1e3) / 1e12
        step_flops = work["index_flops"] + work["main_flops"]
        leg["pipeline"] = {"chunks": max(1, len(runner.chunks)), "streams": 2 if runner.chunks else 1}
        leg["mfma_frac_whole_step"] = step_flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS
        leg["algorithmic_flops_per_step"] = step_flops
        leg["roofline"] = {"bound": "mfma", "stage": dom, "achieved": tf, "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS, "avg_launch_ms": launch_ms,
                           "launches_per_step": launches, "algorithmic_flops_per_launch": algo,
                           "traffic": recorded_traffic(w.name, dom, launches)}
    del runners, runner, inputs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return leg


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3", choices=["c0", "c1", "c2", "c3", "c4d", "c4p", "m3p", "m3d", "c1n", "c2n"])
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (scales PMC byte counters)")
    ap.add_argument("--chunk-rows", type=int, default=65536,
                    help="prefill query rows per pipelined chunk (0: one chunk, no overlap); prefills of at "
                         "most this many rows run unchunked")
    ap.add_argument("--quality-rows", type=int, default=64,
                    help="query rows (evenly spaced) on which to measure selection quality against dense attention; 0: skip")
    ap.add_argument("--dense-calls", type=int, default=3,
                    help="time the dense attention path on the same batch over this many calls after the timed region (0: skip)")
    ap.add_argument("--rotate", type=int, default=None,
                    help="timed steps rotate over this many cache copies (default: 2 for decode, 1 for prefill)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="decode workloads: also time this many single steps, each after a 1 GiB write that evicts the Infinity Cache")
    ap.add_argument("--graph", choices=["on", "off"], default="off",
                    help="replay an unchunked step from a captured HIP graph (stage events then come from a serial pass)")
    ap.add_argument("--legs", default=None,
                    help="comma-separated workloads also measured in the same run after the headline one "
                         "(default with the c3 headline: c1,c4p,c2,c4d, so one run reports prefill and decode at "
                         "128K and 1M; 'none' to skip)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the MSA hot path is not sharded across GPUs (sequences, KV groups "
              "or context blocks would be the shard units). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_long_score_amd import _lib
    from block_sparse_long_score_amd.inputs import WORKLOADS, make_inputs
    from block_sparse_long_score_amd.pipeline import MsaRunner

    _lib.load()  # fails loudly if the HIP library is not built
    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    inputs = make_inputs(w, "cuda")
    runner = MsaRunner(inputs, chunk_rows=args.chunk_rows or None)
    # Decode steps rotate over caches of their own (same contents, separate
    # memory): a step's K_idx and K/V were last touched `rotate` steps ago,
    # with the other copies' traffic (several times the 256 MB Infinity
    # Cache) in between, so no step reads what the previous one left cached.
    n_rot = max(1, args.rotate if args.rotate is not None else (2 if runner.decode else 1))
    runners = [runner] + [MsaRunner(inputs, chunk_rows=args.chunk_rows or None) for _ in range(n_rot - 1)]
    work = algorithmic_work(w)
    stream = torch.cuda.current_stream()

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stages = ("append", "index_score", "block_topk", "attend")
    use_graph = args.graph == "on"
    if use_graph and runner.chunks:
        sys.exit("bench.py: --graph on needs an unchunked step (--chunk-rows 0)")
    steps = [r.step for r in runners]
    if use_graph:
        for r in runners:
            r.capture()
        steps = [r.replay for r in runners]
    step = steps[0]
    for i in range(args.warmup * n_rot):
        steps[i % n_rot]()
    torch.cuda.synchronize()

    def staged_ms():
        """Stage times of the step run serially on one stream, an event after
        each stage (per chunk when chunked); stage time = sum over its launches."""
        out = {k: 0.0 for k in stages}
        marks = []

        def mark(name):
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            marks.append((name, e))

        runner.staged_step(mark)
        torch.cuda.synchronize()
        for (_, e0), (name, e1) in zip(marks, marks[1:]):
            out[name] += e0.elapsed_time(e1)
        return out

    # The dominant stage: decode is bound by the K_idx scan; prefill by
    # whichever of scoring and attention takes longer on this workload.
    pre = staged_ms()
    dom = "index_score" if runner.decode else max(("index_score", "attend"), key=lambda k: pre[k])

    # Timed region: K whole steps (pipelined over two streams when chunked),
    # back to back with an event at each end only.  An event recorded between
    # two kernels leaves a bubble of several microseconds in the stream, which
    # is a tenth of a decode step, so the instrumented timings below come from
    # two more passes of the same K steps in the same run: one with an event
    # between consecutive steps (per-step times for the median) and one with
    # every launch of the dominant stage bracketed by events on the stream it
    # runs on (its live per-launch times, for the roofline).
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_host = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        steps[i % n_rot]()
    end.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # Per-step times (every step ends joined to the caller's stream).
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for i in range(args.steps):
        marks[i].record(stream)
        steps[i % n_rot]()
    marks[-1].record(stream)
    torch.cuda.synchronize()
    step_times = [a.elapsed_time(b) for a, b in zip(marks, marks[1:])]

    # The dominant stage's launches.
    pairs = []

    def hook(name, st, phase):
        if name != dom:
            return
        e = torch.cuda.Event(enable_timing=True)
        e.record(st)
        if phase == 0:
            pairs.append([e, None])
        else:
            pairs[-1][1] = e

    if not use_graph:
        for r in runners:
            r.hook = hook
        for i in range(args.steps):
            runners[i % n_rot].step(fused=False)  # decode: the four calls one by one, so the scan can be bracketed
        torch.cuda.synchronize()
        for r in runners:
            r.hook = None
    if pairs:
        launch_ms = [e0.elapsed_time(e1) for e0, e1 in pairs]
        launches_per_step = len(pairs) / args.steps
    else:  # graph replay: no events inside the graph; serial stage time instead
        launch_ms, launches_per_step = [pre[dom]], 1.0
    avg_launch_ms = sum(launch_ms) / len(launch_ms)

    # Stage breakdown (serial pass), averaged over a few steps.
    n_stage_steps = max(2, min(args.steps, 5))
    stage_ms = {k: 0.0 for k in stages}
    for _ in range(n_stage_steps):
        for k, v in staged_ms().items():
            stage_ms[k] += v / n_stage_steps
    serial_ms = sum(stage_ms.values())

    tokens = w.total_q
    value = tokens / (ms_per_step / 1e3)
    traffic = recorded_traffic(w.name, dom, launches_per_step)
    if runner.decode:
        algo = (work["kidx_bytes"] + work["pooled_bytes"] / 2) / launches_per_step
        achieved = algo / (avg_launch_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "kernel": "msa_index_score (index_score_kernel: K_idx scan + block max-pool)",
                "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": traffic, "algorithmic_bytes_per_launch": algo}
        step_bytes = work["kidx_bytes"] + work["kv_bytes"] + work["io_bytes"] + work["pooled_bytes"]
        step_frac = step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS
        step_info = {"algorithmic_bytes": step_bytes, "hbm_frac_whole_step": step_frac}
    else:
        algo = (work["index_flops"] if dom == "index_score" else work["main_flops"]) / launches_per_step
        achieved = algo / (avg_launch_ms / 1e3) / 1e12
        name = ("msa_index_score (index_score_shared_kernel: scoring + block max-pool)" if dom == "index_score"
                else "msa_sparse_attn_prefill (selection inversion, kvouter_kernel, merge_prefill_kernel)")
        roof = {"bound": "mfma", "kernel": name, "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_PEAK_TFLOPS, "traffic": traffic, "algorithmic_flops_per_launch": algo}
        step_flops = work["index_flops"] + work["main_flops"]
        step_info = {"algorithmic_flops": step_flops,
                     "mfma_frac_whole_step": step_flops / (ms_per_step / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
                     "prefill_tokens_per_s_without_append": tokens / ((ms_per_step - stage_ms["append"]) / 1e3)}
    roof["launches_per_step"] = launches_per_step
    roof["avg_launch_ms"] = avg_launch_ms
    if traffic:  # the stage's measured HBM bytes per launch over its live launch time
        roof["traffic_gbs"] = traffic["bytes_per_launch"] / (avg_launch_ms / 1e3) / 1e9
        roof["traffic_hbm_frac"] = roof["traffic_gbs"] / HBM_PEAK_GBS

    # Single decode steps, each timed right after reading a 1 GiB buffer
    # (outside its events) that evicts the 256 MB Infinity Cache, beside the
    # same isolated steps after reading 1 MiB.  A read evicts without leaving
    # dirty lines whose write-back would load the next step.
    cold = None
    if runner.decode and args.cold_steps > 0:
        def isolated(nbytes):
            buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
            sink = torch.empty((), dtype=torch.float32, device="cuda")
            times = []
            for i in range(args.cold_steps):
                torch.sum(buf, dim=0, out=sink)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                step()
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            return float(np.median(times))
        cold_med = isolated(1 << 30)
        warm_med = isolated(1 << 20)
        cold = {"steps": args.cold_steps, "median_ms_per_step": cold_med, "tokens_per_s": w.total_q / (cold_med / 1e3),
                "evict_read_bytes": 1 << 30, "isolated_after_1mib_read_median_ms": warm_med}

    quality = selection_quality(runner, args.quality_rows) if args.quality_rows > 0 else None
    dense = None
    if args.dense_calls > 0:
        dense = dense_attention(runner, args.dense_calls)
        dense["msa_attend_speedup"] = dense["ms"] / stage_ms["attend"]
        dense["msa_step_speedup"] = dense["ms"] / ms_per_step

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inputs, runner, args.cpu_budget)

    legs_arg = args.legs if args.legs is not None else ("c1,c4p,c2,c4d" if args.workload == "c3" else "none")
    leg_names = [] if legs_arg == "none" else [n for n in legs_arg.split(",") if n and n != args.workload]
    mode = "decode" if runner.decode else "prefill"
    pipeline = {"chunks": max(1, len(runner.chunks)), "streams": 2 if runner.chunks else 1,
                "hip_graph": use_graph, "cache_copies_rotated": n_rot}
    legs = None
    if leg_names:  # the headline workload's buffers are released first
        del runners, runner, steps, step, inputs
        import gc
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        legs = {n: workload_leg(n, args.steps, args.warmup, args.chunk_rows) for n in leg_names}

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "median_ms_per_step": float(np.median(step_times)),
        "timing": {"value": f"{args.steps} steps back to back, events at the two ends only",
                   "median_ms_per_step": f"a second pass of {args.steps} steps, an event between consecutive steps",
                   "roofline": f"a third pass of {args.steps} steps, events around each launch of the dominant stage"
                               + (" (the step's four calls issued one by one instead of msa_decode_step)"
                                  if mode == "decode" else "")},
        "step_calls": ("msa_decode_step (the append fused into the K_idx scan; then selection, attention and "
                       "merge in one kernel below 128 (sequence, group) pairs, else the top-k kernel and the "
                       "attention, two workgroups per pair below 256 pairs)" if mode == "decode" else
                       "msa_kv_append, then per chunk msa_index_score, msa_block_topk, msa_sparse_attn_prefill"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Q/K/V ~ N(0,1) bf16, dyadic-integer Q_idx/K_idx)",
        "config": {"workload": f"{w.name}: {w.description}", "mode": mode,
                   "num_seqs": w.num_seqs, "seq_lens": w.seq_lens[0], "query_tokens_per_step": tokens,
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "index_dim": w.index_dim, "block_size": w.block_size, "top_k": w.top_k},
        "stage_ms": stage_ms,
        "serial_ms_per_step": serial_ms,
        "pipeline": pipeline,
        "step": step_info,
        "roofline": roof,
        "cpu_baseline": cpu,
        "selection_quality": quality,
        "cold_cache": cold,
        "dense_attention": dense,
        "legs": legs,
        "host_wall_s_timed_region": t_host,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
