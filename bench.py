#!/usr/bin/env python3
"""Benchmark of the IndexPool indexer + block-sparse attention path on one MI355X.

One step = one pass of the whole path over one batch:
  decode:  append each sequence's new token to the caches and pool the block it
           completes, score every earlier pooled block and select the top-k (one
           launch: the append rides in the scoring launch and the last scoring
           workgroup of each row selects it), attend over the selected tokens
           (sparse_attn_decode);
  prefill: pool the chunk's new blocks, score and select for every query token
           (scoring launch + selection launch), sparse_attn_prefill;
  IndexCache group (decode_indexcache): the decode step of the group's first DSA
           layer, then for each other layer of the group its new latent row
           (indexpool_append without indexer state) and its attention over the
           first layer's selection; `value` counts (query token, layer) pairs.
The headline workload is decode of 8 sequences x 131072 tokens with top-512 blocks
(2048 tokens).  Inputs are seeded synthetic data of the workload's shape, resident
in HBM before timing; R replicas of every device buffer are rotated so that
successive steps do not hit in the 256 MB last-level cache.  Each replica's step is
captured once into a HIP graph and replayed (--eager launches every call from
Python instead).

Two timed regions of K steps each:
  1. the graph replays -> `value` (query tokens per second) and `ms_per_step`;
  2. the same K steps launched call by call, every kernel launch carrying a pair
     of HIP events that receive its dispatch start and end times
     (hipExtLaunchKernelGGL, on the stream the kernel runs on) -> the per-kernel
     averages in `kernels`, `kernel_sum_ms` and `roofline`.  These are the same
     timestamps rocprofv3's kernel trace reports.
`roofline` for decode is the path: the step's algorithmic bytes (what the method
must move: pooled keys, queries, selected ids, gathered latent rows, outputs and
the cache growth; no score workspace or split partials) over the summed average
durations of the path's kernels, against 8 TB/s; for prefill it is the attention
kernel's FLOPs against the 2.5 PFLOP/s bf16 MFMA peak.  Without --workload the
line also carries `configs`: the same measurement (fewer steps) on the tiny fp32
decode, the chunked prefill, the 1M-token decode and the ragged paged decode.
`cpu_baseline` times the CPU oracle on a bounded sample of the headline workload.
Prints one JSON line.
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
      attention + |U|*dk*2 (gathered latent rows, |U| = selected tokens <= p;
                            |U|*(dk + 4) for the fp8 latent tier: codes + scale)
                + H*dk*2 + H*dv*2     bf16 query in, bf16 output
                + k*4                 ids read
    plus, for decode, each sequence's cache growth: the new token's latent row, key
    and logit read and written, and its completed block pooled (3 cached tokens read,
    one pooled row written); for prefill the pooling of the chunk's new blocks,
    4*(D_I + 4 + 4) read + (D_I + 4) written per block.
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
    row_b = (w.dk + 4) if w.latent_fp8 else w.dk * 2
    attn_b = U * row_b + H * w.dk * 2 + H * w.dv * 2 + k * 4
    sel_b = k * 4
    fp8 = inp.idx_scale is not None
    kv_in = kv_out = 0
    if w.mode == "decode":
        kv_in = w.dk * (2 if w.attn_dtype == "bf16" else 4) + (0 if w.attn_dtype == "bf16" else w.dv * 4)
        kv_out = (w.dk + 4) if w.latent_fp8 else kv_in                # fp8 tier: codes + scale
        key_in, key_out = (D * 2, D + 4) if fp8 else (D * 4, D * 4)
        tok_b = 3 * ((D + 4) if fp8 else D * 4) + 3 * 4          # cached tokens of the block
        grow = kv_in + kv_out + key_in + key_out + 4 + 4 + tok_b + key_out
        pool_b = len(inp.seq_lens) * grow
    else:
        pool_b = (w.n_query // 4) * (4 * (D + 4 + 4) + D + 4)
    # an IndexCache follower layer: its new latent row written, then attention over the
    # first layer's selection (ids read again), no indexer traffic
    fol_b = attn_b.sum() + (len(inp.seq_lens) * (kv_in + kv_out) if w.mode == "decode" else 0)
    return dict(score=int(score_b.sum()), select=int(sel_b * len(n)), attention=int(attn_b.sum()),
                pool=int(pool_b), total=int(score_b.sum() + sel_b * len(n) + attn_b.sum() + pool_b),
                follower=int(fol_b), U=U)


def kernel_bytes(inp, w, ab, fused, step=False):
    """Algorithmic bytes per kernel (the same units as the step total; split
    partials and the score workspace are not counted).  fused: the scoring launch
    also selects (and, for decode, appends); step: one launch does all of that and
    the attention (then only the split combine follows)."""
    n = len(inp.q_pos)
    sel_b = ab["select"]
    if step:
        return {"step": ab["score"] + ab["pool"] + sel_b + ab["attention"], "combine": 0}
    if w.mode == "decode":
        out = {"score": ab["score"] + ab["pool"] + (sel_b if fused else 0), "attention": ab["attention"]}
    else:
        out = {"compress": ab["pool"], "score": ab["score"] + (sel_b if fused else 0), "attention": ab["attention"]}
    if not fused:
        out["topk"] = sel_b
    from long_context_sparse_19_amd import _lib
    part = _lib.LIB.sparse_attn_workspace_bytes(n, w.n_heads, w.dv, w.top_k,
                                                _lib.IP_BF16 if w.attn_dtype == "bf16" else _lib.IP_F32)
    if part:
        out["combine"] = 0          # merges split partials: no algorithmic bytes of its own
    return out


def step_fused(w):
    """Whether indexpool_decode_step runs as one launch (plus the split combine) for
    this workload: decode over fp8 indexer keys and a bf16 latent cache, rows short
    enough for the selection's per-wave lists (fewer than 64 rows), with the
    attention split (the plan of sparse_attn_workspace_bytes) into splits of fewer
    than 128 blocks."""
    if not (w.mode == "decode" and w.idx_key_dtype == "fp8" and w.attn_dtype == "bf16" and not w.latent_fp8):
        return False
    n, k = w.batch, w.top_k
    # the scoring's per-wave lists: 8 per 1024 blocks, at most 256 per row
    if 8 * ((max(1, (w.seq_len - 1) // 4) + 1023) // 1024) > 256 or n >= 64:
        return False
    nsub = (k + 15) // 16
    ns = max(1, min((128 + n - 1) // n, nsub, 64))
    bps = min((nsub + ns - 1) // ns, 32) * 16
    return (k + bps - 1) // bps > 1 and bps < 128


def fuses_select(w):
    """Whether index_score_topk selects inside the scoring launch for this workload
    (fp8 keys and decode-shaped rows: fewer than 64 rows, or no per-row sequence
    table)."""
    return w.idx_key_dtype == "fp8" and w.mode == "decode"


# the sources each kernel is built from (the HBM counters in profiles/ are tied to them)
_KERNEL_SOURCES = {"attention": ("attn.hip", "attn_bf16.hpp", "attn_pipe.hip", "attn_common.hpp"),
                   "combine": ("attn.hip", "attn_bf16.hpp", "attn_common.hpp"),
                   "step": ("attn.hip", "attn_bf16.hpp", "attn_step_h32.hip", "attn_common.hpp", "score_fp8.hpp",
                            "select.hpp"),
                   "score": ("score.hip", "score_fp8.hpp", "select.hpp"), "topk": ("topk.hip", "select.hip", "select.hpp"), "compress": ("compress.hip",),
                   "append": ("compress.hip",), "kda": ("kda.hip",)}


def _source_hash(kind):
    import hashlib
    h = hashlib.sha256()
    for f in (*_KERNEL_SOURCES[kind], "common.hpp", "kernels.hpp", "append.hpp"):
        with open(os.path.join(ROOT, "long_context_sparse_19_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kind, workload):
    """HBM bytes per dispatch of `kind` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (scaled by the copy-kernel calibration), or None when there is
    no record or the kernel's sources changed since the counters were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as fh:
            rec = json.load(fh)[workload]["kernels"][kind]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != _source_hash(kind):
        return None
    return rec["bytes_per_dispatch"]


def attention_flops(U, w):
    return int(2 * w.n_heads * (w.dk + w.dv) * U.sum())


def indexer_flops(inp, w):
    """Dense indexer work: 2 * H_I * D_I flop per (query row, eligible block)."""
    import numpy as np
    n = inp.q_pos.astype(np.int64) // 4
    return int(2 * w.idx_heads * w.idx_dim * n.sum())


def path_traffic(path, workload):
    """Counted HBM bytes of one step's path kernels (sum over them), or None when any
    is missing or stale."""
    tot = 0.0
    for n in path:
        t = measured_traffic(n, workload)
        if t is None:
            return None
        tot += t
    return tot


def cpu_baseline(inp, w, budget_s=12.0, followers=()):
    """The oracle's step (decode: append the new token and pool its block; prefill:
    pool the row's block; then score, select, attend) on whole query rows of the
    same workload, for about budget_s seconds of CPU time."""
    import numpy as np
    from oracle import oracle as O
    from long_context_sparse_19_amd.inputs import new_tokens
    new = new_tokens(w, len(inp.seq_lens), seed=w.seed) if w.mode == "decode" else None
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
            if new is not None:
                O.append(inp, new["kv_new"], new["key_new"], new["logit_new"], only={b})
            else:
                prow = O.pooled_rows(inp, b, np.array([b_q]))
                tok = 4 * prow[:, None] + np.arange(4)[None]
                if inp.idx_scale is not None:
                    O.pool_fp8(inp.idx_keys[tok], inp.idx_scale[tok], inp.pool_logits[tok])
            keys = vals[O.pooled_rows(inp, b, np.arange(b_q))]
            S = O.score(O._to_f64(inp.q_idx[r]), inp.gates[r], keys)
            ids = O.select(S, b_q, w.top_k)
            O.attention_rows(inp, ids[None], w.scale, w.dv, rows=[r])
            for f in followers:      # IndexCache: the other layers over the same ids
                if new is not None:
                    O.append(f, new["kv_new"], new["key_new"], new["logit_new"], only={b})
                O.attention_rows(f, ids[None], w.scale, w.dv, rows=[r])
            done += w.layers
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "query-tokens/s", "cores": blas_threads,
            "kind": "oracle", "host_cores_available": cores,
            "sample": f"{done} (query row, layer) pairs of the {w.name} workload (sequences {seqs}), oracle cache growth / "
                      f"pooling of the new block + float64 scoring over every earlier block + selection + attention, "
                      f"{dt:.1f} s"}


def copy_probe(mb):
    """Ten copies of `mb` MB between two device buffers: a kernel whose HBM traffic
    is known exactly (mb MB read + mb MB written per copy), for scaling the
    FETCH_SIZE / WRITE_SIZE counters of a kernel trace."""
    import torch
    n = mb * 1000 * 1000
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(10):
        flush.fill_(0)               # evicts src / dst from the last-level cache
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 10}))


KDA_METRIC = "KDA decode tokens/s + achieved HBM GB/s (linear-attention state step, 64 heads x 128^2 fp32 state)"


def kda_bytes(kw):
    """Algorithmic bytes of one KDA decode step.  Per (sequence, head): the 128 x 128
    fp32 state read and written, x_q / x_k / x_v (3 x 128 bf16), alpha (128 fp32),
    beta, the conv state (3 x 3 x 128 fp32) read and written, the output (128 fp32);
    per head once: the conv weights (3 x 128 x 4 fp32)."""
    d = kw.head_dim
    per = 2 * d * d * 4 + 3 * d * 2 + d * 4 + 4 + 2 * 9 * d * 4 + d * 4
    return kw.batch * kw.heads * per + kw.heads * 3 * d * 4 * 4


def kda_cpu_baseline(kin, kw, budget_s=12.0):
    """The oracle's decode step on whole sequences for about budget_s of CPU time."""
    import numpy as np
    from oracle import kda as K
    from long_context_sparse_19_amd.inputs import bf16_bits_to_f32
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b = done % kw.batch
        K.decode_step(kin["state"][b:b + 1], kin["conv_state"][b:b + 1], bf16_bits_to_f32(kin["xq"][0][b:b + 1]),
                      bf16_bits_to_f32(kin["xk"][0][b:b + 1]), bf16_bits_to_f32(kin["xv"][0][b:b + 1]),
                      kin["alpha"][0][b:b + 1], kin["beta"][0][b:b + 1], kin["conv_w"])
        done += 1
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": blas_threads, "kind": "oracle",
            "host_cores_available": len(os.sched_getaffinity(0)),
            "sample": f"{done} sequence steps of the {kw.name} workload (all {kw.heads} heads, float64), {dt:.1f} s"}


def kda_main(args, kw):
    """KDA decode step: every timed step updates the state of all sequences and heads
    in place; R state replicas rotate so that successive steps miss the 256 MB cache."""
    import numpy as np
    import torch
    from long_context_sparse_19_amd import _lib, device as D
    from long_context_sparse_19_amd.inputs import kda_inputs
    kin = kda_inputs(kw, 1)
    nbytes = kda_bytes(kw)
    R = args.replicas or max(1, min(32, math.ceil((1 << 30) / nbytes)))
    reps = [D.KdaDevice(kin) for _ in range(R)]
    torch.cuda.synchronize()
    K = args.steps
    graph = None
    if not args.eager:
        # the K timed steps in one HIP graph (one kernel per step: replaying a graph
        # per step would leave the GPU waiting on the host)
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for d in reps:
                d.step(0, alternate=False)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(K):
                reps[(args.warmup + i) % R].step(0, alternate=False)
        torch.cuda.synchronize()

    for i in range(args.warmup):
        reps[i % R].step(0, alternate=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(K):
            reps[(args.warmup + i) % R].step(0, alternate=False)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for e0, e1 in ev:
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    for i in range(K):
        _lib.time_next_launch(_lib.K_KDA, *ev[i])
        reps[(args.warmup + i) % R].step(0, alternate=False)
    torch.cuda.synchronize()
    kt = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    ach = nbytes / (kt * 1e-3) / 1e9
    line = {
        "metric": KDA_METRIC, "value": kw.batch / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": kw.name, "batch": kw.batch, "heads": kw.heads, "head_dim": kw.head_dim,
                   "state": "fp32", "replicas": R, "launch": "eager" if args.eager else "hip-graph",
                   "parallelism": "single GPU"},
        "algorithmic_bytes_per_step": nbytes,
        "hbm_gbps": nbytes / (ms * 1e-3) / 1e9,
        "kernels": {"kda": {"avg_ms": kt, "bytes": nbytes, "GBps": ach}},
        "roofline": {"bound": "hbm", "kernel": "kda_decode_kernel", "achieved": ach, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS, "traffic": measured_traffic("kda", kw.name),
                     "avg_ms": kt, "launches": K},
        "cpu_baseline": None if args.no_cpu_baseline else kda_cpu_baseline(kin, kw),
    }
    return line


KDA_PREFILL_METRIC = "KDA prefill tokens/s (chunked gated delta rule, 64 heads x 128^2 fp32 state)"
FP32_PEAK_TFLOPS = 157.3


def kda_prefill_flops(kw):
    """Algorithmic flops of a KDA prefill chunk: per (token, head) the recurrence's
    three dense products with the 128 x 128 state (S'^T k, the rank-1 write, S^T q),
    2 d^2 each."""
    return 6 * kw.head_dim * kw.head_dim * kw.tokens * kw.heads * kw.batch


def kda_prefill_main(args, kw):
    """KDA prefill: every timed step runs the whole chunk (kda_prefill_chunk) on the
    state in place."""
    import numpy as np
    import torch
    from long_context_sparse_19_amd import _lib, device as D
    from long_context_sparse_19_amd.inputs import kda_inputs
    kin = kda_inputs(kw, kw.tokens)
    d = D.KdaChunkDevice(kin)
    torch.cuda.synchronize()
    K = args.steps
    for _ in range(args.warmup):
        d.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        d.run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for e0, e1 in ev:
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    for i in range(K):
        _lib.time_next_launch(_lib.K_KDA, *ev[i])
        d.run()
    torch.cuda.synchronize()
    kt = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    fl = kda_prefill_flops(kw)
    ach = fl / (kt * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import kda as Ko
        from long_context_sparse_19_amd.inputs import bf16_bits_to_f32
        n = min(kw.tokens, 256)
        sw = lambda x: np.swapaxes(x[:n], 0, 1)
        tc = time.perf_counter()
        Ko.prefill_chunk(kin["state"], kin["conv_state"], sw(bf16_bits_to_f32(kin["xq"])), sw(bf16_bits_to_f32(kin["xk"])),
                         sw(bf16_bits_to_f32(kin["xv"])), sw(kin["alpha"]), sw(kin["beta"]), kin["conv_w"])
        dt = time.perf_counter() - tc
        cpu = {"value": kw.batch * n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "host_cores_available": len(os.sched_getaffinity(0)),
               "sample": f"the first {n} tokens of the chunk, token by token (all {kw.heads} heads, float64), {dt:.1f} s"}
    line = {
        "metric": KDA_PREFILL_METRIC, "value": kw.batch * kw.tokens / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": kw.name, "batch": kw.batch, "tokens": kw.tokens, "heads": kw.heads,
                   "head_dim": kw.head_dim, "state": "fp32", "launch": "eager", "parallelism": "single GPU"},
        "algorithmic_flops_per_step": fl,
        "kernels": {"kda_chunk": {"avg_ms": kt, "flops": fl, "TFLOPs": ach}},
        "roofline": {"bound": "mfma", "kernel": "kda_chunk_kernel", "achieved": ach, "peak": FP32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": ach / FP32_PEAK_TFLOPS, "traffic": None, "avg_ms": kt, "launches": K},
        "cpu_baseline": cpu,
    }
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    from long_context_sparse_19_amd.configs import WORKLOADS as _W, KDA_WORKLOADS as _KW
    ap.add_argument("--workload", default="decode", choices=list(_W) + list(_KW))
    ap.add_argument("--replicas", type=int, default=0, help="rotated input copies (0 = auto, >= 1 GiB touched)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="headline workload only (no `configs` key)")
    ap.add_argument("--eager", action="store_true", help="launch every call from Python instead of HIP graphs")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only run 10 plain device copies of MB megabytes (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode (got --gpus {args.gpus}); "
              f"sharding across GPUs is described in the design notes but not built.", file=sys.stderr)
        sys.exit(2)

    if args.workload in _KW:
        kw = _KW[args.workload]
        print(json.dumps((kda_prefill_main if kw.tokens else kda_main)(args, kw)))
        return

    from long_context_sparse_19_amd.configs import WORKLOADS
    w = WORKLOADS[args.workload]
    res, line = run_workload(w, args.steps, args.warmup, args.replicas, args.eager, with_cpu=not args.no_cpu_baseline)
    if args.workload == "decode" and not args.no_configs:
        # the other configurations, fewer steps each: tiny fp32 decode, chunked
        # prefill, 1M-token decode, ragged paged decode
        extra = {}
        for name in ("tiny", "prefill", "max_ctx", "ragged"):
            steps = max(3, min(args.steps, 10))
            r, _ = run_workload(WORKLOADS[name], steps, 2, 2 if name != "max_ctx" else 1, args.eager, with_cpu=False)
            extra[name] = r
        # the KDA half of the hybrid layer: a decode step and a 4096-token prefill chunk
        from long_context_sparse_19_amd.configs import KDA_WORKLOADS
        for name, kw in KDA_WORKLOADS.items():
            ka = argparse.Namespace(**{**vars(args), "steps": max(3, min(args.steps, 10)), "warmup": 2,
                                       "no_cpu_baseline": True, "replicas": 0})
            kl = (kda_prefill_main if kw.tokens else kda_main)(ka, kw)
            extra[name] = {"workload": name, "ms_per_step": kl["ms_per_step"], "value": kl["value"], "unit": kl["unit"],
                           "roofline": kl["roofline"], "kernels": kl["kernels"], "steps": kl["steps"]}
        line["configs"] = extra
    print(json.dumps(line))


def run_workload(w, K, warmup, replicas, eager, with_cpu):
    """Times workload w; returns (a summary dict, the full JSON line)."""
    import numpy as np
    import torch
    from long_context_sparse_19_amd import _lib, device as D
    from long_context_sparse_19_amd.inputs import make_inputs, new_tokens, follower_layer

    t_gen = time.perf_counter()
    inp = make_inputs(w)
    # IndexCache: the group's other DSA layers (own latent cache and queries, no indexer)
    followers = [follower_layer(inp, l) for l in range(1, w.layers)]
    print(f"[bench] {w.name}: inputs drawn in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    ab = algorithmic_bytes(inp, w)
    step_bytes = ab["total"] + len(followers) * ab["follower"]
    R = replicas or max(1, min(32 // w.layers, math.ceil((1 << 30) / max(1, step_bytes))))
    base = D.upload(inp)
    reps = [base]
    for _ in range(R - 1):
        reps.append(D.DeviceInputs(**{**base.__dict__,
                                      "keys": _lib.Cache(base.keys.data.clone(), None if base.keys.scale is None else base.keys.scale.clone()),
                                      "logits": base.logits.clone(),
                                      "pooled": _lib.Cache(base.pooled.data.clone(), None if base.pooled.scale is None else base.pooled.scale.clone()),
                                      "kv": _lib.Cache(base.kv.data.clone(), None if base.kv.scale is None else base.kv.scale.clone()),
                                      "v": None if base.v is None else _lib.Cache(base.v.data.clone()),
                                      "q": base.q.clone(), "q_idx": base.q_idx.clone(), "gates": base.gates.clone()}))
    for d in reps:
        D.compress(d)            # cache build (untimed)
    fbase = [D.upload_follower(f, base) for f in followers]
    freps = [fbase] + [[D.DeviceInputs(**{**fd.__dict__, "seqs": reps[i].seqs,
                                           "kv": _lib.Cache(fd.kv.data.clone(), None if fd.kv.scale is None else fd.kv.scale.clone()),
                                           "q": fd.q.clone()}) for fd in fbase] for i in range(1, R)]
    # prefill keeps its whole score matrix (one pass over the 8192 rows; the
    # library otherwise scores in passes of at most 256 MB)
    wss = [D.Workspaces(d, keep_scores=(w.mode == "prefill")) for d in reps]
    fwss = [[D.FollowerWorkspaces(fd, wss[i]) for fd in freps[i]] for i in range(R)]
    if w.mode == "decode":
        # each sequence's new token (at seq_lens - 1, the query position)
        toks = D.NewTokens(new_tokens(w, len(inp.seq_lens), seed=w.seed))
    else:
        begin = torch.full((1,), int(inp.q_pos[0]) // 4, dtype=torch.int32, device="cuda")
        max_new = (int(inp.q_pos[-1]) // 4) - (int(inp.q_pos[0]) // 4) + 1
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: {R} replicas resident, {step_bytes / 1e6:.2f} MB algorithmic per step", file=sys.stderr,
          flush=True)

    def step(i):
        d, ws = reps[i % R], wss[i % R]
        if w.mode == "decode":
            D.decode_step(d, toks, ws)           # append + score + top-k + attention
        else:
            D.compress(d, block_begin=begin, max_blocks=max_new)
            D.score_topk(d, ws)
            D.attention(d, ws)
        for fd, fws in zip(freps[i % R], fwss[i % R]):
            D.append(fd, toks)
            D.attention(fd, fws)

    graphs = None
    if not eager:
        # one HIP graph per replica holding one whole step
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for i in range(R):
                step(i)            # warm once outside capture
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        for i in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        # and one graph holding a step on every replica in turn, as a serving loop
        # launches many steps at once
        gall = None
        if R > 1:
            gall = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gall):
                for i in range(R):
                    step(i)
        torch.cuda.synchronize()

    def run_steps(i, n):
        """Steps i .. i+n-1, step j on replica j mod R."""
        end = i + n
        while i < end:
            if graphs is None:
                step(i % R)
                i += 1
            elif gall is not None and i % R == 0 and end - i >= R:
                gall.replay()
                i += R
            else:
                graphs[i % R].replay()
                i += 1

    # --- timed region 1: K whole steps -> value (the warm-up ends on the replica
    # before the first timed one)
    run_steps(-warmup, warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(0, K)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / K
    value = w.n_rows * w.layers / (ms / 1e3)     # (query token, DSA layer) pairs per second

    # --- timed region 2: the same K steps launched one call at a time, every kernel
    # launch carrying HIP events that receive its dispatch start / end times (the
    # timestamps a kernel trace reports), on the stream the kernel runs on
    fused = fuses_select(w)
    kbytes = kernel_bytes(inp, w, ab, fused, step=step_fused(w))
    ids = {"compress": _lib.K_COMPRESS, "score": _lib.K_SCORE, "topk": _lib.K_TOPK, "attention": _lib.K_ATTN,
           "combine": _lib.K_COMBINE, "step": _lib.K_STEP}
    ids = {n: kid for n, kid in ids.items() if n in kbytes}     # the kernels this workload launches
    evk = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
           for n in ids}
    for n in ids:
        for e0, e1 in evk[n]:
            e0.record()
            e1.record()            # materialise the events before handing them to the library
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(K):
        for n, kid in ids.items():
            _lib.time_next_launch(kid, *evk[n][i])
        step(warmup + i)
    torch.cuda.synchronize()
    _lib.time_next_launch(0, None, None)          # disarm what a step did not consume
    eager_ms = (time.perf_counter() - t1) * 1e3 / K
    kern_ms = {}
    for n in ids:
        ts = [e0.elapsed_time(e1) for e0, e1 in evk[n]]
        ts = [t for t in ts if t > 0]
        if len(ts) == K:
            kern_ms[n] = float(np.mean(ts))

    U = ab["U"]
    kernels = {}
    for n, t in kern_ms.items():
        # prefill rows share their keys and latent rows: per-row gathered bytes are
        # no HBM figure there, its scoring and attention are priced in flops
        b = None if (w.mode == "prefill" and n in ("score", "attention")) else kbytes.get(n)
        kernels[n] = {"avg_ms": t, "bytes": b, "GBps": (b / (t * 1e-3) / 1e9) if b else None,
                      "hbm_frac": (b / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS) if b else None}
    if "attention" in kernels:
        fl = attention_flops(U, w)
        tf = fl / (kern_ms["attention"] * 1e-3) / 1e12
        kernels["attention"].update(flops=fl, TFLOPs=tf, mfma_frac=tf / BF16_PEAK_TFLOPS)
    if w.mode == "prefill" and "score" in kernels:
        ifl = indexer_flops(inp, w)
        tf = ifl / (kern_ms["score"] * 1e-3) / 1e12
        kernels["score"].update(flops=ifl, TFLOPs=tf, mfma_frac=tf / BF16_PEAK_TFLOPS)
    path = [n for n in ("step", "score", "topk", "attention", "combine") if n in kern_ms]
    path_ms = sum(kern_ms[n] for n in path)
    if w.mode == "prefill":
        ach = kernels["attention"]["TFLOPs"]
        roof = {"bound": "mfma", "kernel": "attention (sparse_attn_prefill)", "achieved": ach,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                "traffic": measured_traffic("attention", w.name), "avg_ms": kern_ms["attention"], "launches": K}
    else:
        ach = step_bytes / (path_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "decode path: " + " + ".join(path), "achieved": ach, "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS, "traffic": path_traffic(path, w.name),
                "avg_ms": path_ms, "launches": K}

    cpu = cpu_baseline(inp, w, followers=followers) if with_cpu else None
    summary = {"workload": w.name, "ms_per_step": ms, "value": value, "unit": "query-tokens/s",
               "kernel_sum_ms": path_ms, "roofline": roof, "kernels": kernels, "steps": K, "replicas": R}
    if w.mode == "prefill":
        summary["attention_flops_per_step"] = attention_flops(U, w)
        summary["indexer_flops_per_step"] = indexer_flops(inp, w)
    else:
        summary["algorithmic_bytes_per_step"] = step_bytes
    line = {
        "metric": METRIC, "value": value, "unit": "query-tokens/s", "n_gpus": 1, "steps": K,
        "warmup": warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.attn_dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "context": w.seq_len, "query_rows": w.n_rows,
                   "top_k_blocks": w.top_k, "index_keys": w.idx_key_dtype, "latent": "fp8" if w.latent_fp8 else w.attn_dtype,
                   "dsa_layers": w.layers, "replicas": R, "launch": "eager" if eager else "hip-graph",
                   "parallelism": "single GPU"},
        "hbm_gbps": step_bytes / (ms * 1e-3) / 1e9,
        "algorithmic_bytes_per_step": step_bytes,
        "kernel_sum_ms": path_ms,
        "hbm_frac_kernel_sum": step_bytes / (path_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS if path_ms else None,
        "eager_ms_per_step": eager_ms,
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    del reps, freps, wss, fwss, graphs
    torch.cuda.empty_cache()
    return summary, line


if __name__ == "__main__":
    main()
