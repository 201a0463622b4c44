"""Phase timeline of the fused decode step (the decode workload: 8 sequences x 131072
tokens), from the stamps of the diagnostics library:

    python -m long_context_sparse_19_amd.build --stamps
    python -m long_context_sparse_19_amd.phase_timeline [--rounds 10]

Each round launches 6 steps back to back (on rotating input replicas, so that steps do
not hit in the last-level cache) and reads the stamps of the last one.  Times are µs
from the first workgroup's start of that step; each line gives the minimum, median and
maximum over the workgroups of a role and over the rounds."""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

os.environ["IP_LIBRARY"] = "stamps"

import numpy as np  # noqa: E402
import torch  # noqa: E402

from long_context_sparse_19_amd import _lib, device as D  # noqa: E402
from long_context_sparse_19_amd.configs import DECODE  # noqa: E402
from long_context_sparse_19_amd.inputs import make_inputs, new_tokens  # noqa: E402

SLOTS, STEP_ROWS, ROWS = 8, 4096, 5120


def replicas(inp, n):
    base = D.upload(inp)
    reps = [base]
    for _ in range(n - 1):
        reps.append(D.DeviceInputs(**{
            **base.__dict__,
            "keys": _lib.Cache(base.keys.data.clone(), base.keys.scale.clone()),
            "logits": base.logits.clone(),
            "pooled": _lib.Cache(base.pooled.data.clone(), base.pooled.scale.clone()),
            "kv": _lib.Cache(base.kv.data.clone()),
            "q": base.q.clone(), "q_idx": base.q_idx.clone(), "gates": base.gates.clone()}))
    return reps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--rounds", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=8)
    args = ap.parse_args()
    w = DECODE
    inp = make_inputs(w)
    reps = replicas(inp, args.replicas)
    for d in reps:
        D.compress(d)
    wss = [D.Workspaces(d) for d in reps]
    toks = D.NewTokens(new_tokens(w, len(inp.seq_lens), seed=w.seed))
    buf = np.zeros(ROWS * SLOTS, dtype=np.uint64)
    # the step's workgroups: scoring (one row of gx per sequence), append, attention
    gx = (int(inp.seq_lens.max() - 1) // 4 + 1023) // 1024
    n_score, n_app = gx * w.batch, w.batch
    acc = {}
    it = 0
    for _ in range(args.rounds):
        for _ in range(6):
            D.decode_step(reps[it % len(reps)], toks, wss[it % len(reps)])
            it += 1
        torch.cuda.synchronize()
        _lib._check("ip_phase_stamps", _lib.LIB.ip_phase_stamps(buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes))
        b = buf.reshape(ROWS, SLOTS).astype(np.int64)
        sc, at = b[:n_score], b[n_score + n_app:STEP_ROWS]
        at = at[at[:, 0] > 0]
        cb = b[STEP_ROWS:]
        cb = cb[cb[:, 0] > 0]
        t0 = min(sc[:, 0].min(), at[:, 0].min())
        us = lambda v: (v - t0) / 100.0   # 100 MHz ticks -> µs
        for name, v in (("scoring: start", sc[:, 0]), ("scoring: scores and lists stored", sc[:, 1]),
                        ("attention: start", at[:, 0]), ("attention: ids ready (lists merged)", at[:, 2]),
                        ("attention: sub-tile 0 landed", at[:, 3]), ("attention: sub-tiles done", at[:, 4]),
                        ("attention: partials stored", at[:, 5]), ("combine: start", cb[:, 0]),
                        ("combine: end", cb[:, 1])):
            acc.setdefault(name, []).append(us(v))
    print(f"fused decode step, {w.batch} x {w.seq_len} tokens: µs from the first workgroup's start "
          f"(min / median / max over workgroups and {args.rounds} steps)")
    for name, v in acc.items():
        x = np.concatenate(v)
        print(f"  {name:38s} {x.min():7.2f} {np.median(x):7.2f} {x.max():7.2f}")


if __name__ == "__main__":
    sys.exit(main())
