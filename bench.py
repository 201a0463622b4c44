#!/usr/bin/env python3
"""Benchmark of the IndexPool indexer + block-sparse attention path on one MI355X.

One step = one pass of the whole path over one batch:
  decode:  pool the block each query just completed (indexpool_compress), score
           every earlier pooled block and select the top-k (index_score_topk),
           attend over the selected tokens (sparse_attn_decode);
  prefill: pool the chunk's new blocks, score/select for every query token,
           sparse_attn_prefill.
The default workload is decode of 8 sequences x 131072 tokens with top-512
blocks (2048 tokens).  Inputs are seeded synthetic data of the workload's shape,
resident in HBM before timing; R replicas of every device buffer are rotated so
that successive steps do not hit in the 256 MB last-level cache.  Each replica's
step is captured once into a HIP graph and replayed (--eager launches every call
from Python instead).

Prints one JSON line.  `value` is query tokens per second; `hbm_gbps` the
algorithmic bytes of a step over the step time; `roofline` describes the
dominant kernel with its average duration from HIP events recorded around its
launches inside the timed region; `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode query-tokens/s + achieved HBM GB/s (indexer+sparse attn) at 128K ctx"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def algorithmic_bytes(inp, w):
    """Bytes the method itself must move per step (no workspace, no partials).

    Per query row with n = b_q eligible blocks:
      scoring   n*(D_I + 4)          pooled fp8 codes + fp32 scale
                + H_I*D_I*2 + H_I*4   bf16 query, fp32 gates
      selection k*4                  ids written
      attention + |U|*dk*2 (gathered latent rows, |U| = selected tokens <= p)
                + H*dk*2 + H*dv*2     bf16 query in, bf16 output
                + k*4                 ids read
    plus the pooling of the new blocks: 4*(D_I + 4 + 4) read + (D_I + 4) written per block.
    """
    import numpy as np
    D, HI, H = w.idx_dim, w.idx_heads, w.n_heads
    n = inp.q_pos.astype(np.int64) // 4
    k = w.top_k
    kp = np.minimum(k, n + 1)
    # tokens of the selected blocks: all 4 of every block except the own one
    own = inp.q_pos.astype(np.int64) % 4 + 1
    U = (kp - 1) * 4 + own
    score_b = n * (D + 4) + HI * D * 2 + HI * 4
    attn_b = U * w.dk * 2 + H * w.dk * 2 + H * w.dv * 2 + k * 4
    sel_b = k * 4
    new_blocks = len(inp.seq_lens) if w.mode == "decode" else w.n_query // 4
    pool_b = new_blocks * (4 * (D + 4 + 4) + D + 4)
    return dict(score=int(score_b.sum()), select=int(sel_b * len(n)), attention=int(attn_b.sum()),
                pool=int(pool_b), total=int(score_b.sum() + sel_b * len(n) + attn_b.sum() + pool_b),
                U=U)


def attention_flops(U, w):
    return int(2 * w.n_heads * (w.dk + w.dv) * U.sum())


def cpu_baseline(inp, w, budget_s=12.0):
    """The oracle's step (pool the new block, score, select, attend) on whole query
    rows of the same workload, for about budget_s seconds of CPU time."""
    import numpy as np
    from oracle import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    rows = list(range(w.n_rows))
    # the cache build (pooling every complete block before the step) is untimed;
    # only the sequences of the sampled rows are pooled
    seqs = sorted({int(inp.q_seq[r]) for r in rows[: min(len(rows), 2)]})
    sample_rows = [r for r in rows if int(inp.q_seq[r]) in seqs][:64]
    D = inp.idx_keys.shape[1]
    vals = np.zeros((inp.n_rows_tok // 4, D))
    for b in seqs:
        nb = int(inp.seq_lens[b]) // 4
        prow = O.pooled_rows(inp, b, np.arange(nb))
        tok = 4 * prow[:, None] + np.arange(4)[None]
        if inp.idx_scale is None:
            vals[prow] = O.pool_f32(inp.idx_keys[tok], inp.pool_logits[tok])
        else:
            c, s, _, _ = O.pool_fp8(inp.idx_keys[tok], inp.idx_scale[tok], inp.pool_logits[tok])
            vals[prow] = O.pooled_values(c, s)
    done = 0
    t0 = time.perf_counter()
    while True:
        for r in sample_rows:
            b = int(inp.q_seq[r])
            p = int(inp.q_pos[r])
            b_q = p // 4
            prow = O.pooled_rows(inp, b, np.array([b_q]))
            tok = 4 * prow[:, None] + np.arange(4)[None]
            if inp.idx_scale is not None:
                O.pool_fp8(inp.idx_keys[tok], inp.idx_scale[tok], inp.pool_logits[tok])
            keys = vals[O.pooled_rows(inp, b, np.arange(b_q))]
            S = O.score(O._to_f64(inp.q_idx[r]), inp.gates[r], keys)
            ids = O.select(S, b_q, w.top_k)
            O.attention_rows(inp, ids[None], w.scale, w.dv, rows=[r])
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "query-tokens/s", "cores": blas_threads,
            "kind": "oracle", "host_cores_available": cores,
            "sample": f"{done} query rows of the {w.name} workload (sequences {seqs}), oracle pooling of the "
                      f"new block + float64 scoring over every earlier block + selection + attention, "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["decode", "max_ctx", "ragged", "prefill", "tiny"])
    ap.add_argument("--replicas", type=int, default=0, help="rotated input copies (0 = auto, >= 1 GiB touched)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch every call from Python instead of HIP graphs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode (got --gpus {args.gpus}); "
              f"sharding across GPUs is described in the design notes but not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from long_context_sparse_19_amd import _lib, device as D
    from long_context_sparse_19_amd.configs import WORKLOADS
    from long_context_sparse_19_amd.inputs import make_inputs

    w = WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    inp = make_inputs(w)
    print(f"[bench] {w.name}: inputs drawn in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    ab = algorithmic_bytes(inp, w)
    step_bytes = ab["total"]
    R = args.replicas or max(1, min(32, math.ceil((1 << 30) / max(1, step_bytes))))
    base = D.upload(inp)
    reps = [base]
    for _ in range(R - 1):
        reps.append(D.DeviceInputs(**{**base.__dict__,
                                      "keys": _lib.Cache(base.keys.data.clone(), None if base.keys.scale is None else base.keys.scale.clone()),
                                      "logits": base.logits.clone(),
                                      "pooled": _lib.Cache(base.pooled.data.clone(), None if base.pooled.scale is None else base.pooled.scale.clone()),
                                      "kv": _lib.Cache(base.kv.data.clone()),
                                      "v": None if base.v is None else _lib.Cache(base.v.data.clone()),
                                      "q": base.q.clone(), "q_idx": base.q_idx.clone(), "gates": base.gates.clone()}))
    for d in reps:
        D.compress(d)            # cache build (untimed)
    wss = [D.Workspaces(d) for d in reps]
    if w.mode == "decode":
        begin = torch.from_numpy((inp.q_pos // 4).astype(np.int32)).cuda()
        max_new = 1
    else:
        begin = torch.full((1,), int(inp.q_pos[0]) // 4, dtype=torch.int32, device="cuda")
        max_new = (int(inp.q_pos[-1]) // 4) - (int(inp.q_pos[0]) // 4) + 1
    torch.cuda.synchronize()
    print(f"[bench] {R} replicas resident, {step_bytes / 1e6:.2f} MB algorithmic per step", file=sys.stderr, flush=True)

    def step(i, ev=None):
        d, ws = reps[i % R], wss[i % R]
        D.compress(d, block_begin=begin, max_blocks=max_new)
        if ev is not None:
            _lib.time_next_launch(_lib.K_SCORE, ev[0], ev[1])
        D.score_topk(d, ws)
        if ev is not None:
            _lib.time_next_launch(_lib.K_ATTN, ev[2], ev[3])
        D.attention(d, ws)

    # per-replica events around the score and attention kernels
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(R)]
    for e in evs:
        for x in e:
            x.record()             # materialise the events before handing them to the library
    torch.cuda.synchronize()

    graphs = None
    if not args.eager:
        # one HIP graph per replica holding one whole step (the library only
        # enqueues kernels and event records on the capturing stream)
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(R):
                step(i)            # warm once outside capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for i in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i, evs[i])
            graphs.append(g)
        torch.cuda.synchronize()

    def run(i, timed):
        if graphs is not None:
            graphs[i % R].replay()
        else:
            step(i, evs[i % R] if timed else None)

    for i in range(args.warmup):
        run(i, False)
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for i in range(K):
        run(args.warmup + i, True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    used = sorted({(args.warmup + i) % R for i in range(K)})
    score_ms = float(np.mean([evs[j][0].elapsed_time(evs[j][1]) for j in used]))
    attn_ms = float(np.mean([evs[j][2].elapsed_time(evs[j][3]) for j in used]))
    ms = dt * 1e3 / K
    value = w.n_rows / (ms / 1e3)

    U = ab["U"]
    score_bytes = ab["score"]
    attn_bytes = ab["attention"]
    kernels = {
        "score": {"avg_ms": score_ms, "algorithmic_bytes": score_bytes,
                  "GBps": score_bytes / (score_ms * 1e-3) / 1e9},
        "attention": {"avg_ms": attn_ms, "algorithmic_bytes": attn_bytes,
                      "GBps": attn_bytes / (attn_ms * 1e-3) / 1e9,
                      "flops": attention_flops(U, w),
                      "TFLOPs": attention_flops(U, w) / (attn_ms * 1e-3) / 1e12},
    }
    if w.mode == "prefill":
        ach = kernels["attention"]["TFLOPs"]
        roof = {"bound": "mfma", "kernel": "attn_bf16 (sparse_attn_prefill)", "achieved": ach,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS, "traffic": None}
    else:
        name, kk = max(kernels.items(), key=lambda kv: kv[1]["avg_ms"])
        ach = kk["GBps"]
        roof = {"bound": "hbm", "kernel": name, "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBPS, "traffic": None}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, w)

    line = {
        "metric": METRIC, "value": value, "unit": "query-tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "context": w.seq_len, "query_rows": w.n_rows,
                   "top_k_blocks": w.top_k, "index_keys": w.idx_key_dtype, "latent": w.attn_dtype,
                   "replicas": R, "launch": "eager" if args.eager else "hip-graph",
                   "parallelism": "single GPU"},
        "hbm_gbps": step_bytes / (ms * 1e-3) / 1e9,
        "algorithmic_bytes_per_step": step_bytes,
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
