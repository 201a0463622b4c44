"""Seeded synthetic inputs for every workload.

This module only draws random numbers and lays them out; it holds none of the
pooling, scoring, selection or attention arithmetic.  Both the device path (tests,
bench) and the CPU oracle consume the arrays it returns, so both see the same
bytes.

Recipe (numpy PCG64; every array has its own seed stream derived from the
workload seed and a fixed tag, and large arrays are drawn in fixed-size row
chunks, so the values do not depend on how much memory is free):

* all values are N(0,1) float32, except the per-head indexer gates, N(0,1)/2;
* one pooling logit per cached token, N(0,1);
* bf16 tensors are the float32 draws rounded to nearest even (torch's cast);
* fp8 index keys: each token row x is stored as codes = e4m3fn(x / s) with the
  per-token scale s = max|x| / 448 (torch's cast, after clamping to +-448);
* salient rows: in each sequence, round(salient_frac * L) token rows drawn
  uniformly without replacement get their index-key scale multiplied by 8
  (their codes are unchanged), which makes the blocks holding them stand out;
* ragged lengths: L_b = 4 * U{min_blocks .. seq_len/4}; the paged cache uses
  64-token pages and one seeded permutation of all pages of all sequences, shared
  by the token-level and the pooled caches.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

from .configs import Workload, KdaWorkload, INDEX_KPOOL

_CHUNK_ROWS = 1 << 16

_TAGS = {
    "lens": 1, "perm": 2, "idx_keys": 3, "logits": 4, "latent": 5, "k": 6, "v": 7,
    "q": 8, "q_idx": 9, "gates": 10, "salient": 11, "append": 12,
    "kda_x": 13, "kda_gate": 14, "kda_state": 15, "kda_conv": 16,
}


def _rng(seed: int, tag: str, chunk: int = 0, layer: int = 0) -> np.random.Generator:
    key = [seed, _TAGS[tag], chunk] + ([layer] if layer else [])
    return np.random.default_rng(np.random.SeedSequence(key))


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _chunked(rows: int, fn) -> None:
    """Run fn(chunk_index, r0, r1) over fixed row chunks on a thread pool (numpy's
    generators and torch's casts release the GIL); results do not depend on the
    thread count because every chunk has its own seed stream."""
    spans = [(c, r0, min(rows, r0 + _CHUNK_ROWS)) for c, r0 in enumerate(range(0, rows, _CHUNK_ROWS))]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda a: fn(*a), spans))


def _normal_rows(seed: int, tag: str, rows: int, cols: int, layer: int = 0) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)

    def fill(c, r0, r1):
        _rng(seed, tag, c, layer).standard_normal((r1 - r0, cols), dtype=np.float32, out=out[r0:r1])
    _chunked(rows, fill)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (torch's cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _fp8_span(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row fp8 e4m3fn storage of float32 rows (codes, scale = amax / 448) using
    torch's cast; runs on the calling thread."""
    import torch
    amax = np.abs(x).max(axis=1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s_safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    y = torch.from_numpy(np.ascontiguousarray(x)) / torch.from_numpy(s_safe[:, None])
    return y.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy(), s


def _fp8_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """_fp8_span over row chunks on the thread pool."""
    codes = np.empty(x.shape, dtype=np.uint8)
    s = np.empty(x.shape[0], dtype=np.float32)

    def conv(c, r0, r1):
        codes[r0:r1], s[r0:r1] = _fp8_span(x[r0:r1])
    _chunked(x.shape[0], conv)
    return codes, s


@dataclass
class Inputs:
    w: Workload
    seq_lens: np.ndarray            # int32 [B] tokens
    page_table: Optional[np.ndarray]  # int32 [B, max_pages] or None
    page_tokens: int                # tokens per page (0 if contiguous)
    seq_stride: int                 # tokens between sequences (contiguous layout)
    n_rows_tok: int                 # physical token rows
    idx_keys: np.ndarray            # uint8 fp8 codes [R, D_I] or float32 [R, D_I]
    idx_scale: Optional[np.ndarray]  # float32 [R] (fp8 keys) or None
    pool_logits: np.ndarray         # float32 [R]
    latent: Optional[np.ndarray]    # uint16 bf16 bits [R, dk] (bf16 workloads), or uint8
                                    # fp8 e4m3fn codes with latent_scale (fp8 latent tier)
    k_cache: Optional[np.ndarray]   # float32 [R, dk] (f32 workload)
    v_cache: Optional[np.ndarray]   # float32 [R, dv] (f32 workload)
    q: np.ndarray                   # uint16 bf16 bits or float32 [n_q, H, dk]
    q_idx: np.ndarray               # uint16 bf16 bits or float32 [n_q, H_I, D_I]
    gates: np.ndarray               # float32 [n_q, H_I]
    q_seq: np.ndarray               # int32 [n_q]
    q_pos: np.ndarray               # int32 [n_q]
    salient_rows: np.ndarray        # int64 physical token rows whose scale was x8
    latent_scale: Optional[np.ndarray] = None   # float32 [R] (fp8 latent tier)

    @property
    def max_pages(self) -> int:
        return 0 if self.page_table is None else int(self.page_table.shape[1])

    @property
    def n_rows_pooled(self) -> int:
        return self.n_rows_tok // INDEX_KPOOL


def _attention_cache(w: Workload, n_rows: int, layer: int):
    """The latent cache of one DSA layer (bf16 bits, or fp8 codes + per-token scale),
    or the float K and V caches of the f32 workload."""
    seed = w.seed
    latent = latent_scale = k_cache = v_cache = None
    if w.attn_dtype == "bf16" and w.latent_fp8:
        # fp8 latent tier: the same N(0,1) rows stored as e4m3fn codes with a
        # per-token scale (amax / 448)
        latent = np.empty((n_rows, w.dk), dtype=np.uint8)
        latent_scale = np.empty(n_rows, dtype=np.float32)

        def fill8(c, r0, r1):
            x = _rng(seed, "latent", c, layer).standard_normal((r1 - r0, w.dk), dtype=np.float32)
            latent[r0:r1], latent_scale[r0:r1] = _fp8_span(x)
        _chunked(n_rows, fill8)
    elif w.attn_dtype == "bf16":
        latent = np.empty((n_rows, w.dk), dtype=np.uint16)

        def fill(c, r0, r1):
            latent[r0:r1] = to_bf16_bits(
                _rng(seed, "latent", c, layer).standard_normal((r1 - r0, w.dk), dtype=np.float32))
        _chunked(n_rows, fill)
    else:
        k_cache = _normal_rows(seed, "k", n_rows, w.dk, layer)
        v_cache = _normal_rows(seed, "v", n_rows, w.dv, layer)
    return latent, latent_scale, k_cache, v_cache


def _query_rows(w: Workload, n_q: int, layer: int) -> np.ndarray:
    return _normal_rows(w.seed, "q", n_q, w.n_heads * w.dk, layer).reshape(n_q, w.n_heads, w.dk)


def follower_layer(inp: "Inputs", layer: int) -> "Inputs":
    """DSA layer `layer` (>= 1) of an IndexCache group whose first layer is `inp`: the
    same sequences and query positions, its own latent cache and attention queries,
    and no indexer state (it attends over the first layer's selection)."""
    w = inp.w
    latent, latent_scale, k_cache, v_cache = _attention_cache(w, inp.n_rows_tok, layer)
    qf = _query_rows(w, len(inp.q_pos), layer)
    q = to_bf16_bits(qf) if w.attn_dtype == "bf16" else qf
    return replace(inp, idx_keys=None, idx_scale=None, pool_logits=None, q_idx=None, gates=None,
                   latent=latent, latent_scale=latent_scale, k_cache=k_cache, v_cache=v_cache, q=q,
                   salient_rows=np.zeros(0, dtype=np.int64))


def make_inputs(w: Workload, with_attention: bool = True) -> Inputs:
    """Draw every input of workload ``w`` (host numpy arrays)."""
    B = w.batch
    seed = w.seed
    if w.ragged:
        nb = _rng(seed, "lens").integers(w.min_blocks, w.seq_len // INDEX_KPOOL + 1, size=B)
        seq_lens = (nb * INDEX_KPOOL).astype(np.int32)
    else:
        seq_lens = np.full(B, w.seq_len, dtype=np.int32)

    page_table = None
    if w.page_tokens:
        pt = w.page_tokens
        assert pt % INDEX_KPOOL == 0
        n_pages = (seq_lens.astype(np.int64) + pt - 1) // pt
        total = int(n_pages.sum())
        perm = _rng(seed, "perm").permutation(total).astype(np.int32)
        max_pages = int(n_pages.max())
        page_table = np.zeros((B, max_pages), dtype=np.int32)
        off = 0
        for b in range(B):
            page_table[b, : n_pages[b]] = perm[off: off + n_pages[b]]
            off += int(n_pages[b])
        n_rows = total * pt
        seq_stride = 0
    else:
        seq_stride = int(w.seq_len)
        n_rows = B * seq_stride

    # token rows of every (sequence, token) in the physical cache, for salient rows
    def phys_rows(b: int, t: np.ndarray) -> np.ndarray:
        if page_table is None:
            return b * seq_stride + t
        return page_table[b, t // w.page_tokens].astype(np.int64) * w.page_tokens + t % w.page_tokens

    # indexer keys
    x = _normal_rows(seed, "idx_keys", n_rows, w.idx_dim)
    if w.idx_key_dtype == "fp8":
        idx_keys, idx_scale = _fp8_rows(x)
    else:
        idx_keys, idx_scale = x, None
    del x
    salient = np.zeros(0, dtype=np.int64)
    if w.salient_frac > 0 and idx_scale is not None:
        rs = _rng(seed, "salient")
        picks = []
        for b in range(B):
            L = int(seq_lens[b])
            n = int(round(w.salient_frac * L))
            t = rs.choice(L, size=n, replace=False)
            picks.append(phys_rows(b, np.sort(t)))
        salient = np.concatenate(picks)
        idx_scale[salient] *= np.float32(w.salient_mult)
    logits = _normal_rows(seed, "logits", n_rows, 1)[:, 0].copy()

    # attention caches
    latent = k_cache = v_cache = latent_scale = None
    if with_attention:
        latent, latent_scale, k_cache, v_cache = _attention_cache(w, n_rows, 0)

    # queries
    n_q = w.n_rows
    if w.mode == "decode":
        q_seq = np.arange(B, dtype=np.int32)
        q_pos = (seq_lens - 1).astype(np.int32)
    else:
        assert B == 1
        q_seq = np.zeros(n_q, dtype=np.int32)
        q_pos = (int(seq_lens[0]) - n_q + np.arange(n_q)).astype(np.int32)
    qf = _query_rows(w, n_q, 0)
    qif = _normal_rows(seed, "q_idx", n_q, w.idx_heads * w.idx_dim).reshape(n_q, w.idx_heads, w.idx_dim)
    gates = (_normal_rows(seed, "gates", n_q, w.idx_heads) * np.float32(0.5)).astype(np.float32)
    if w.attn_dtype == "bf16":
        q = to_bf16_bits(qf)
        q_idx = to_bf16_bits(qif)
    else:
        q, q_idx = qf, qif

    return Inputs(
        w=w, seq_lens=seq_lens, page_table=page_table, page_tokens=w.page_tokens,
        seq_stride=seq_stride, n_rows_tok=n_rows, idx_keys=idx_keys, idx_scale=idx_scale,
        pool_logits=logits, latent=latent, k_cache=k_cache, v_cache=v_cache, q=q,
        q_idx=q_idx, gates=gates, q_seq=q_seq, q_pos=q_pos, salient_rows=salient,
        latent_scale=latent_scale,
    )


def new_tokens(w: Workload, batch: int, seed: int) -> dict:
    """One decode step's new token per sequence, seeded N(0,1) like the caches:
    kv_new (bf16 bits [B, dk] latent rows, or float32 K rows), v_new (float32 [B, dv]
    or None), key_new (bf16 bits [B, D_I] for fp8 key caches, float32 otherwise) and
    logit_new (float32 [B])."""
    rng = _rng(seed, "append")
    bf16 = w.attn_dtype == "bf16"
    kv = rng.standard_normal((batch, w.dk), dtype=np.float32)
    key = rng.standard_normal((batch, w.idx_dim), dtype=np.float32)
    return {
        "kv_new": to_bf16_bits(kv) if bf16 else kv,
        "v_new": None if bf16 else rng.standard_normal((batch, w.dv), dtype=np.float32),
        "key_new": to_bf16_bits(key) if w.idx_key_dtype == "fp8" else key,
        "logit_new": rng.standard_normal(batch, dtype=np.float32),
    }


def kda_inputs(kw: KdaWorkload, steps: int = 1) -> dict:
    """Seeded inputs of `steps` KDA decode steps.  Per step t: xq, xk, xv (bf16 bits
    [B, H*d], N(0,1)), alpha = sigmoid(N(0,1) + 3) per key channel (a slow decay,
    about 0.95) and beta = sigmoid(N(0,1)) per head.  Shared: conv_w N(0,1)/2
    [3, H*d, 4], the initial state N(0,1)/sqrt(d) [B, H, d, d] and the initial conv
    state N(0,1) [B, 3, 3, H*d], all float32."""
    B, H, d = kw.batch, kw.heads, kw.head_dim
    seed = kw.seed
    x = _normal_rows(seed, "kda_x", steps * 3 * B, H * d).reshape(steps, 3, B, H * d)
    g = _rng(seed, "kda_gate")
    alpha = (1.0 / (1.0 + np.exp(-(g.standard_normal((steps, B, H, d), dtype=np.float32) + 3.0)))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-g.standard_normal((steps, B, H), dtype=np.float32)))).astype(np.float32)
    c = _rng(seed, "kda_conv")
    conv_w = (c.standard_normal((3, H * d, 4), dtype=np.float32) * np.float32(0.5)).astype(np.float32)
    conv_state = c.standard_normal((B, 3, 3, H * d), dtype=np.float32)
    state = (_normal_rows(seed, "kda_state", B * H * d, d) * np.float32(1.0 / np.sqrt(d))).reshape(B, H, d, d)
    return {"xq": to_bf16_bits(x[:, 0]), "xk": to_bf16_bits(x[:, 1]), "xv": to_bf16_bits(x[:, 2]),
            "alpha": alpha, "beta": beta, "conv_w": conv_w, "conv_state": conv_state, "state": state}

