"""Workload definitions for the IndexPool indexer + block-sparse attention path.

The constants the pages fix:

* ``index_kpool = 4``  -- IndexPool merges four consecutive indexer keys into one
  (G2C Brief "GLM-5.3-Flash: hybrid attention becomes the product", section
  "DSA keeps selected global access in eleven layers"; reading notes
  "GLM-5.3-Flash: Hybrid Attention, IndexPool, and Vision-in-the-Loop", section 2,
  sub-section "IndexPool").
* ``index_topk = 2048`` tokens of selected history per query, i.e. 512 pooled
  blocks of 4 (same G2C section, the pipeline figure and the config fields).
* ``kv_lora_rank = 512`` -- the MLA latent rank per token (same G2C section).

Everything else here (head counts, head sizes, dtypes, lengths, seeds) is the
workload recipe this library is measured on; it is not printed on the pages.
The five workloads are:

* ``tiny``    -- fp32 decode, 1 x 4096 tokens, 16 query heads over one K/V head of
  64 dims, indexer 4 heads x 32 dims, top-64 blocks.
* ``decode``  -- bf16 decode, 8 sequences x 131072 tokens, MQA with 64 heads over a
  576-dim latent row (512 value dims + 64 rope dims), fp8 e4m3fn index keys with a
  per-token fp32 scale, indexer 32 heads x 128 dims, top-512 blocks.
* ``prefill`` -- bf16 chunked prefill: 8192 query tokens appended to a 65536-token
  prefix (73728 tokens in total), top-512 blocks per query token.
* ``max_ctx`` -- bf16 decode of one 1048576-token sequence.
* ``ragged``  -- bf16 decode of 64 sequences of 4096..32768 tokens in a paged cache
  of 64-token pages with a shuffled page table.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

# Constants the pages fix (see the module docstring for where).
INDEX_KPOOL = 4          # tokens per pooled index block
INDEX_TOPK_TOKENS = 2048  # selected tokens per query
KV_LORA_RANK = 512       # latent (value) rank per token
ROPE_DIM = 64            # rope part appended to the latent row (K = 512 + 64)


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str                 # "decode" or "prefill"
    batch: int                # number of sequences
    seq_len: int              # tokens per sequence (upper bound when ragged)
    # attention geometry
    n_heads: int
    dk: int
    dv: int
    attn_dtype: str           # "f32" (separate K and V caches) or "bf16" (one latent row)
    scale: float
    # indexer geometry
    idx_heads: int
    idx_dim: int
    idx_key_dtype: str        # "f32" or "fp8"
    top_k: int                # selected blocks per query (own block included)
    seed: int
    # prefill only: number of query tokens appended at the end of the sequence
    n_query: int = 1
    # ragged decode: lengths drawn as 4*U{min_blocks..max_blocks}
    ragged: bool = False
    min_blocks: int = 0
    page_tokens: int = 0      # 0 = contiguous cache
    salient_frac: float = 0.0  # fraction of index-key rows whose scale is x8
    salient_mult: float = 8.0
    latent_fp8: bool = False  # latent cache in fp8 e4m3fn with a per-token scale
    layers: int = 1           # DSA layers of an IndexCache group (the first runs the indexer)

    @property
    def n_rows(self) -> int:
        """Query rows per step."""
        return self.batch if self.mode == "decode" else self.n_query

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _g1(name: str, **kw) -> Workload:
    base = dict(
        n_heads=64, dk=KV_LORA_RANK + ROPE_DIM, dv=KV_LORA_RANK, attn_dtype="bf16",
        scale=1.0 / (192.0 ** 0.5), idx_heads=32, idx_dim=128, idx_key_dtype="fp8",
        top_k=INDEX_TOPK_TOKENS // INDEX_KPOOL,
    )
    base.update(kw)
    return Workload(name=name, **base)


TINY = Workload(
    name="tiny", mode="decode", batch=1, seq_len=4096, n_heads=16, dk=64, dv=64,
    attn_dtype="f32", scale=1.0 / 8.0, idx_heads=4, idx_dim=32, idx_key_dtype="f32",
    top_k=64, seed=0,
)
DECODE = _g1("decode", mode="decode", batch=8, seq_len=131072, seed=1, salient_frac=0.01)
PREFILL = _g1("prefill", mode="prefill", batch=1, seq_len=73728, n_query=8192, seed=2)
MAX_CTX = _g1("max_ctx", mode="decode", batch=1, seq_len=1048576, seed=3, salient_frac=0.01)
RAGGED = _g1("ragged", mode="decode", batch=64, seq_len=32768, ragged=True,
             min_blocks=1024, page_tokens=64, seed=4)

# The lower-precision latent tier: decode as above over an fp8 latent cache
DECODE_FP8KV = DECODE.with_(name="decode_fp8kv", latent_fp8=True)

# IndexCache: a group of 4 DSA layers, decode as above; the first layer's selection
# serves the other three, which keep no indexer state
DECODE_INDEXCACHE = DECODE.with_(name="decode_indexcache", layers=4)

WORKLOADS = {w.name: w for w in (TINY, DECODE, PREFILL, MAX_CTX, RAGGED, DECODE_FP8KV, DECODE_INDEXCACHE)}


@dataclass(frozen=True)
class KdaWorkload:
    """The linear-attention (KDA) half: 64 heads of width 128 (a 128 x 128 fp32 state
    per head), short convolution of width 4.  tokens = 0: one decode step per
    sequence; tokens > 0: a prefill chunk of that many tokens per sequence."""
    name: str
    batch: int
    heads: int = 64
    head_dim: int = 128
    seed: int = 7
    tokens: int = 0


KDA_DECODE = KdaWorkload("kda_decode", batch=8)
# a 4096-token prefill chunk of one sequence (the chunked form)
KDA_PREFILL = KdaWorkload("kda_prefill", batch=1, tokens=4096, seed=8)
KDA_WORKLOADS = {KDA_DECODE.name: KDA_DECODE, KDA_PREFILL.name: KDA_PREFILL}


def scaled_down(w: Workload, seq_len: int, batch: Optional[int] = None,
                n_query: Optional[int] = None, top_k: Optional[int] = None,
                min_blocks: Optional[int] = None, seed: Optional[int] = None) -> Workload:
    """The same geometry and dtypes at a smaller size (for oracle-sized parity cases)."""
    kw = dict(seq_len=seq_len)
    if batch is not None:
        kw["batch"] = batch
    if n_query is not None:
        kw["n_query"] = n_query
    if top_k is not None:
        kw["top_k"] = top_k
    if min_blocks is not None:
        kw["min_blocks"] = min_blocks
    if seed is not None:
        kw["seed"] = seed
    return w.with_(**kw)
