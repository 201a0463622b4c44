"""Device-resident copies of a workload's inputs and the three-stage pipeline.

Thin glue over the C ABI (``_lib``): it uploads the seeded host arrays once,
allocates outputs and workspaces with torch, and calls indexpool_compress,
index_score_topk and sparse_attn_decode / sparse_attn_prefill.  All arithmetic
runs in the HIP kernels behind those calls.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib
from .inputs import Inputs


def _dev(x: np.ndarray, device, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


@dataclass
class DeviceInputs:
    inp: Inputs
    seqs: _lib.Seqs
    keys: Optional[_lib.Cache]   # token-level index keys (None: an IndexCache follower)
    logits: Optional[torch.Tensor]
    pooled: Optional[_lib.Cache]  # pooled keys (output of compress)
    kv: _lib.Cache            # latent (bf16, or fp8 codes + scales) or K (f32)
    v: Optional[_lib.Cache]   # V (f32 only)
    q: torch.Tensor
    q_idx: Optional[torch.Tensor]
    gates: Optional[torch.Tensor]
    q_seq: torch.Tensor
    q_pos: torch.Tensor
    top_k: int
    scale: float
    dv: int

    @property
    def n_q(self) -> int:
        return self.q.shape[0]

    @property
    def is_decode(self) -> bool:
        return self.inp.w.mode == "decode"


def upload(inp: Inputs, device="cuda") -> DeviceInputs:
    w = inp.w
    seq_lens = _dev(inp.seq_lens, device)
    pt = None if inp.page_table is None else _dev(inp.page_table, device)
    seqs = _lib.Seqs(seq_lens, int(inp.seq_lens.max()), pt, inp.page_tokens, inp.seq_stride)
    R = inp.n_rows_tok
    if inp.idx_scale is not None:
        keys = _lib.Cache(_dev(inp.idx_keys, device), _dev(inp.idx_scale, device))
        pooled = _lib.Cache(torch.zeros((R // 4, inp.idx_keys.shape[1]), dtype=torch.uint8, device=device),
                            torch.zeros(R // 4, dtype=torch.float32, device=device))
    else:
        keys = _lib.Cache(_dev(inp.idx_keys, device))
        pooled = _lib.Cache(torch.zeros((R // 4, inp.idx_keys.shape[1]), dtype=torch.float32, device=device))
    logits = _dev(inp.pool_logits, device)
    kv = v = None
    if w.attn_dtype == "bf16":
        if inp.latent is not None and inp.latent_scale is not None:   # fp8 latent tier
            kv = _lib.Cache(_dev(inp.latent, device), _dev(inp.latent_scale, device))
        elif inp.latent is not None:
            kv = _lib.Cache(_dev(inp.latent, device, torch.bfloat16))
        q = _dev(inp.q, device, torch.bfloat16)
        q_idx = _dev(inp.q_idx, device, torch.bfloat16)
    else:
        if inp.k_cache is not None:
            kv = _lib.Cache(_dev(inp.k_cache, device))
            v = _lib.Cache(_dev(inp.v_cache, device))
        q = _dev(inp.q, device)
        q_idx = _dev(inp.q_idx, device)
    return DeviceInputs(inp=inp, seqs=seqs, keys=keys, logits=logits, pooled=pooled, kv=kv, v=v, q=q,
                        q_idx=q_idx, gates=_dev(inp.gates, device), q_seq=_dev(inp.q_seq, device),
                        q_pos=_dev(inp.q_pos, device), top_k=w.top_k, scale=w.scale, dv=w.dv)


def compress(d: DeviceInputs, block_begin: Optional[torch.Tensor] = None, max_blocks: int = 0,
             stream=None) -> None:
    _lib.indexpool_compress(d.seqs, d.keys, d.logits, d.pooled, block_begin, max_blocks, stream)


class NewTokens:
    """One decode step's new tokens on the device (see inputs.new_tokens)."""

    def __init__(self, new: dict, device="cuda"):
        bf16 = new["kv_new"].dtype == np.uint16
        self.kv_new = _dev(new["kv_new"], device, torch.bfloat16 if bf16 else None)
        self.v_new = None if new["v_new"] is None else _dev(new["v_new"], device)
        kbf16 = new["key_new"].dtype == np.uint16
        self.key_new = _dev(new["key_new"], device, torch.bfloat16 if kbf16 else None)
        self.logit_new = _dev(new["logit_new"], device)


def append(d: DeviceInputs, t: NewTokens, stream=None) -> None:
    """Write each sequence's new token (at seq_lens[b] - 1) and pool a completed block
    (a layer without indexer state: only the latent row)."""
    if d.keys is None:
        _lib.indexpool_append(d.seqs, t.kv_new, d.kv, None, None, None, None, None, v_new=t.v_new, v=d.v,
                              stream=stream)
        return
    _lib.indexpool_append(d.seqs, t.kv_new, d.kv, t.key_new, d.keys, t.logit_new, d.logits, d.pooled,
                          v_new=t.v_new, v=d.v, stream=stream)


def upload_follower(f: Inputs, anchor: DeviceInputs, device="cuda") -> DeviceInputs:
    """An IndexCache follower layer: its own latent cache and queries on the device,
    the anchor's sequences; no indexer state (it attends over the anchor's selection)."""
    w = f.w
    kv = v = None
    if f.latent is not None and f.latent_scale is not None:
        kv = _lib.Cache(_dev(f.latent, device), _dev(f.latent_scale, device))
    elif f.latent is not None:
        kv = _lib.Cache(_dev(f.latent, device, torch.bfloat16))
    else:
        kv = _lib.Cache(_dev(f.k_cache, device))
        v = _lib.Cache(_dev(f.v_cache, device))
    q = _dev(f.q, device, torch.bfloat16 if w.attn_dtype == "bf16" else None)
    return DeviceInputs(inp=f, seqs=anchor.seqs, keys=None, logits=None, pooled=None, kv=kv, v=v, q=q,
                        q_idx=None, gates=None, q_seq=anchor.q_seq, q_pos=anchor.q_pos, top_k=anchor.top_k,
                        scale=anchor.scale, dv=anchor.dv)


class FollowerWorkspaces:
    """Outputs of a follower layer's attention; the selection is the anchor's."""

    def __init__(self, d: DeviceInputs, anchor_ws: "Workspaces"):
        dev = d.q.device
        self.sel = anchor_ws.sel
        qdt = _lib.IP_BF16 if d.q.dtype == torch.bfloat16 else _lib.IP_F32
        na = _lib.sparse_attn_workspace_bytes(d.n_q, d.q.shape[1], d.dv, d.top_k, qdt)
        self.ws_attn = torch.empty(max(na, 16), dtype=torch.uint8, device=dev)
        self.out = torch.empty((d.n_q, d.q.shape[1], d.dv), dtype=d.q.dtype, device=dev)
        self.lse = torch.empty((d.n_q, d.q.shape[1]), dtype=torch.float32, device=dev)
        # the whole decode step's workspace (indexer, attention, ready words), zero-filled
        self.ws_step = None
        if d.is_decode and d.keys is not None:
            ns = _lib.indexpool_decode_step_workspace_bytes(d.seqs, d.top_k, d.q.shape[1], d.dv, qdt, keep_scores)
            self.ws_step = torch.zeros(max(ns, 256), dtype=torch.uint8, device=dev)


class Workspaces:
    """Outputs and workspaces of one pipeline pass, allocated once."""

    def __init__(self, d: DeviceInputs, keep_scores: bool = False):
        dev = d.q.device
        self.sel = torch.empty((d.n_q, d.top_k), dtype=torch.int32, device=dev)
        self.scores = None
        if keep_scores:
            ld = _lib.index_scores_ld(d.seqs.max_seq_len)
            self.scores = torch.zeros((d.n_q, ld), dtype=torch.float32, device=dev)
        nb = _lib.index_score_topk_workspace_bytes(d.seqs, d.n_q, d.top_k, keep_scores)
        # zero-filled once: the fused selection's per-row counters start at zero and
        # every call leaves them there
        self.ws_idx = torch.zeros(max(nb, 256), dtype=torch.uint8, device=dev)
        qdt = _lib.IP_BF16 if d.q.dtype == torch.bfloat16 else _lib.IP_F32
        na = _lib.sparse_attn_workspace_bytes(d.n_q, d.q.shape[1], d.dv, d.top_k, qdt)
        self.ws_attn = torch.empty(max(na, 16), dtype=torch.uint8, device=dev)
        self.out = torch.empty((d.n_q, d.q.shape[1], d.dv), dtype=d.q.dtype, device=dev)
        self.lse = torch.empty((d.n_q, d.q.shape[1]), dtype=torch.float32, device=dev)
        # the whole decode step's workspace (indexer, attention, ready words), zero-filled
        self.ws_step = None
        if d.is_decode and d.keys is not None:
            ns = _lib.indexpool_decode_step_workspace_bytes(d.seqs, d.top_k, d.q.shape[1], d.dv, qdt, keep_scores)
            self.ws_step = torch.zeros(max(ns, 256), dtype=torch.uint8, device=dev)


def score_topk(d: DeviceInputs, ws: Workspaces, stream=None) -> None:
    q_seq = None if d.is_decode else d.q_seq
    q_pos = None if d.is_decode else d.q_pos
    _lib.index_score_topk(d.seqs, d.q_idx, d.gates, d.pooled, d.top_k, ws.sel, q_seq=q_seq, q_pos=q_pos,
                          scores=ws.scores, ws=ws.ws_idx, stream=stream)


def decode_index(d: DeviceInputs, t: NewTokens, ws: Workspaces, stream=None) -> None:
    """append(d, t) then score_topk(d, ws) for the decode rows, in one call (the
    append rides in the scoring launch)."""
    _lib.indexpool_decode_index(d.seqs, t.kv_new, d.kv, t.key_new, d.keys, t.logit_new, d.logits, d.pooled,
                                d.q_idx, d.gates, d.top_k, ws.sel, scores=ws.scores, ws=ws.ws_idx, v_new=t.v_new,
                                v=d.v, stream=stream)


def decode_step(d: DeviceInputs, t: NewTokens, ws: Workspaces, stream=None) -> None:
    """decode_index(d, t, ws) then attention(d, ws), in one call (one launch plus the
    split combine where the geometry allows)."""
    _lib.indexpool_decode_step(d.seqs, t.kv_new, d.kv, t.key_new, d.keys, t.logit_new, d.logits, d.pooled,
                               d.q_idx, d.gates, d.top_k, ws.sel, d.q, ws.out, d.scale, d.dv, lse=ws.lse,
                               scores=ws.scores, ws=ws.ws_step, v_new=t.v_new, v=d.v, stream=stream)


def attention(d: DeviceInputs, ws: Workspaces, sel: Optional[torch.Tensor] = None, stream=None) -> None:
    sel = ws.sel if sel is None else sel
    if d.is_decode:
        _lib.sparse_attn_decode(d.seqs, d.q, d.kv, d.v, sel, ws.out, d.scale, d.dv, lse=ws.lse,
                                ws=ws.ws_attn, stream=stream)
    else:
        _lib.sparse_attn_prefill(d.seqs, d.q, d.kv, d.v, sel, ws.out, d.scale, d.dv, d.q_seq, d.q_pos,
                                 lse=ws.lse, ws=ws.ws_attn, stream=stream)


class KdaDevice:
    """Device copies of KDA decode inputs (inputs.kda_inputs): per-step x / alpha /
    beta, the conv weights, and the state and conv state that each step updates."""

    def __init__(self, kin: dict, device="cuda"):
        self.xq = _dev(kin["xq"], device, torch.bfloat16)
        self.xk = _dev(kin["xk"], device, torch.bfloat16)
        self.xv = _dev(kin["xv"], device, torch.bfloat16)
        self.alpha = _dev(kin["alpha"], device)
        self.beta = _dev(kin["beta"], device)
        self.conv_w = _dev(kin["conv_w"], device)
        self.conv = [_dev(kin["conv_state"], device), torch.empty_like(_dev(kin["conv_state"], device))]
        self.parity = 0               # conv[parity] holds the current taps
        self.state = _dev(kin["state"], device)
        B, H, d = self.state.shape[0], self.state.shape[1], self.state.shape[3]
        self.out = torch.empty((B, H, d), dtype=torch.float32, device=device)

    @property
    def conv_state(self) -> torch.Tensor:
        return self.conv[self.parity]

    def step(self, t: int, stream=None, alternate: bool = True) -> None:
        """Step t's inputs; the conv taps move to the other buffer, which becomes
        the current one (alternate=False keeps reading the same buffer, for
        repeated timing of one step)."""
        _lib.kda_decode_step(self.xq[t], self.xk[t], self.xv[t], self.alpha[t], self.beta[t], self.conv_w,
                             self.conv[self.parity], self.conv[1 - self.parity], self.state, self.out,
                             stream=stream)
        if alternate:
            self.parity = 1 - self.parity


class KdaChunkDevice:
    """Device copies of the inputs of one KDA prefill chunk of T tokens (from
    inputs.kda_inputs with steps = T, token-major there, sequence-major here)."""

    def __init__(self, kin: dict, device="cuda"):
        tr = lambda x: np.ascontiguousarray(np.swapaxes(x, 0, 1))
        self.xq = _dev(tr(kin["xq"]), device, torch.bfloat16)
        self.xk = _dev(tr(kin["xk"]), device, torch.bfloat16)
        self.xv = _dev(tr(kin["xv"]), device, torch.bfloat16)
        self.alpha = _dev(tr(kin["alpha"]), device)
        self.beta = _dev(tr(kin["beta"]), device)
        self.conv_w = _dev(kin["conv_w"], device)
        self.conv_in = _dev(kin["conv_state"], device)
        self.conv_out = torch.empty_like(self.conv_in)
        self.state = _dev(kin["state"], device)
        B, T = self.xq.shape[0], self.xq.shape[1]
        H, d = self.state.shape[1], self.state.shape[3]
        self.out = torch.empty((B, T, H, d), dtype=torch.float32, device=device)

    def run(self, stream=None) -> None:
        _lib.kda_prefill_chunk(self.xq, self.xk, self.xv, self.alpha, self.beta, self.conv_w, self.conv_in,
                               self.conv_out, self.state, self.out, stream=stream)
