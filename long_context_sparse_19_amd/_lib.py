"""ctypes binding of libindexpool.so (argument marshalling only).

Every function here turns torch tensors into device pointers and forwards to the
C entry point of the same name; no step of the computation runs in Python.  The
library must have been built (``python -m long_context_sparse_19_amd.build``);
importing this module without it raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# IP_LIBRARY=stamps loads the diagnostics build that records the decode step's phase
# stamps (libindexpool_stamps.so, `python -m long_context_sparse_19_amd.build --stamps`)
LIB_PATH = os.path.join(_PKG, "libindexpool_stamps.so" if os.environ.get("IP_LIBRARY") == "stamps"
                        else "libindexpool.so")

IP_OK, IP_EINVAL, IP_EUNSUPPORTED, IP_EWORKSPACE, IP_EDEVICE = range(5)
IP_F32, IP_BF16, IP_FP8_E4M3FN = range(3)
K_COMPRESS, K_SCORE, K_TOPK, K_ATTN, K_COMBINE, K_APPEND, K_KDA, K_STEP = 1, 2, 3, 4, 5, 6, 7, 8

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_size = ctypes.c_size_t


class IpCache(ctypes.Structure):
    _fields_ = [("data", _c_void_p), ("scale", _c_void_p), ("dtype", _i32),
                ("row_dim", _i32), ("row_stride", _i64)]


class IpSeqs(ctypes.Structure):
    _fields_ = [("batch", _i32), ("max_seq_len", _i32), ("seq_lens", _c_void_p),
                ("page_table", _c_void_p), ("max_pages", _i32), ("page_tokens", _i32),
                ("seq_stride", _i64)]


class IndexPoolError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> status {status}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m long_context_sparse_19_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.indexpool_compress.argtypes = [P(IpSeqs), _c_void_p, _i32, P(IpCache), _c_void_p, P(IpCache), _c_void_p]
    lib.indexpool_append.argtypes = [P(IpSeqs), _c_void_p, P(IpCache), _c_void_p, P(IpCache), _c_void_p, _i32,
                                     P(IpCache), _c_void_p, _c_void_p, P(IpCache), _c_void_p]
    lib.index_scores_ld.argtypes = [_i32]
    lib.index_scores_ld.restype = _i64
    lib.index_score_topk_workspace_bytes.argtypes = [P(IpSeqs), _i32, _i32, _i32]
    lib.index_score_topk_workspace_bytes.restype = _size
    lib.index_score_topk.argtypes = [P(IpSeqs), _i32, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                     _c_void_p, P(IpCache), _i32, _c_void_p, _c_void_p, _c_void_p, _size,
                                     _c_void_p]
    lib.index_score_topk_noalloc.argtypes = [P(IpSeqs), _i32, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                             _c_void_p, P(IpCache), _i32, _c_void_p, _c_void_p, _c_void_p]
    lib.index_score_topk_noalloc_max_bytes.argtypes = []
    lib.index_score_topk_noalloc_max_bytes.restype = _size
    lib.sparse_attn_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32]
    lib.sparse_attn_workspace_bytes.restype = _size
    lib.sparse_attn_decode.argtypes = [P(IpSeqs), _c_void_p, _i32, _i32, _i32, _i32, ctypes.c_float,
                                       P(IpCache), P(IpCache), _c_void_p, _i32, _c_void_p, _c_void_p,
                                       _c_void_p, _size, _c_void_p]
    lib.sparse_attn_prefill.argtypes = [P(IpSeqs), _i32, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                        _i32, ctypes.c_float, P(IpCache), P(IpCache), _c_void_p, _i32,
                                        _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]
    lib.indexpool_decode_index.argtypes = [P(IpSeqs), _c_void_p, P(IpCache), _c_void_p, P(IpCache), _c_void_p, _i32,
                                           P(IpCache), _c_void_p, _c_void_p, P(IpCache), _c_void_p, _i32, _i32, _i32,
                                           _c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]
    lib.indexpool_decode_step_workspace_bytes.argtypes = [P(IpSeqs), _i32, _i32, _i32, _i32, _i32]
    lib.indexpool_decode_step_workspace_bytes.restype = _size
    lib.indexpool_decode_step.argtypes = [P(IpSeqs), _c_void_p, P(IpCache), _c_void_p, P(IpCache), _c_void_p, _i32,
                                          P(IpCache), _c_void_p, _c_void_p, P(IpCache), _c_void_p, _i32, _i32, _i32,
                                          _c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32,
                                          ctypes.c_float, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]
    lib.kda_decode_step.argtypes = [_i32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p,
                                    _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]
    lib.kda_prefill_chunk.argtypes = [_i32, _i32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p,
                                      _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]
    lib.ip_last_error.restype = ctypes.c_char_p
    lib.ip_version.restype = ctypes.c_char_p
    lib.ip_time_next_launch.argtypes = [_i32, _c_void_p, _c_void_p]
    lib.ip_phase_stamps.argtypes = [_c_void_p, _size]
    for fn in ("indexpool_compress", "indexpool_append", "index_score_topk", "indexpool_decode_index",
               "indexpool_decode_step", "sparse_attn_decode", "sparse_attn_prefill", "kda_decode_step",
               "kda_prefill_chunk", "ip_time_next_launch", "ip_phase_stamps"):
        getattr(lib, fn).restype = ctypes.c_int
    return lib


LIB = _load()

EXPORTED = ("indexpool_compress", "indexpool_append", "indexpool_decode_index", "indexpool_decode_step",
            "indexpool_decode_step_workspace_bytes", "index_scores_ld", "index_score_topk_workspace_bytes", "index_score_topk",
            "index_score_topk_noalloc", "index_score_topk_noalloc_max_bytes",
            "sparse_attn_workspace_bytes", "sparse_attn_decode", "sparse_attn_prefill", "kda_decode_step",
            "kda_prefill_chunk", "ip_last_error",
            "ip_time_next_launch", "ip_phase_stamps", "ip_version")


def _check(fn: str, st: int) -> None:
    if st != IP_OK:
        raise IndexPoolError(fn, st, LIB.ip_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


_DT = {torch.float32: IP_F32, torch.bfloat16: IP_BF16, torch.uint8: IP_FP8_E4M3FN,
       torch.float8_e4m3fn: IP_FP8_E4M3FN}


@dataclass
class Cache:
    """A cache of rows: ``data`` [rows, row_dim] (uint8 codes for fp8) + fp8 scale."""
    data: torch.Tensor
    scale: Optional[torch.Tensor] = None

    def c(self) -> IpCache:
        d = self.data
        return IpCache(d.data_ptr(), _ptr(self.scale), _DT[d.dtype], d.shape[1], d.stride(0) * d.element_size())


@dataclass
class Seqs:
    """Sequences of a batch: device seq_lens (+ page table) and the host bound."""
    seq_lens: torch.Tensor
    max_seq_len: int
    page_table: Optional[torch.Tensor] = None
    page_tokens: int = 0
    seq_stride: int = 0

    def c(self) -> IpSeqs:
        mp = 0 if self.page_table is None else self.page_table.shape[1]
        return IpSeqs(self.seq_lens.shape[0], self.max_seq_len, self.seq_lens.data_ptr(),
                      _ptr(self.page_table), mp, self.page_tokens, self.seq_stride)


def indexpool_compress(seqs: Seqs, keys: Cache, logits: torch.Tensor, pooled: Cache,
                       block_begin: Optional[torch.Tensor] = None, max_blocks: int = 0, stream=None) -> None:
    s, k, p = seqs.c(), keys.c(), pooled.c()
    _check("indexpool_compress", LIB.indexpool_compress(
        ctypes.byref(s), _ptr(block_begin), max_blocks, ctypes.byref(k), logits.data_ptr(), ctypes.byref(p),
        _stream(stream)))


def indexpool_append(seqs: Seqs, kv_new: torch.Tensor, kv: Cache, key_new: Optional[torch.Tensor],
                     keys: Optional[Cache], logit_new: Optional[torch.Tensor], logits: Optional[torch.Tensor],
                     pooled: Optional[Cache], v_new: Optional[torch.Tensor] = None, v: Optional[Cache] = None,
                     stream=None) -> None:
    """keys (with key_new, logit_new, logits, pooled) None: a layer without indexer
    state, only kv (and v) rows are written."""
    s, kc = seqs.c(), kv.c()
    k = None if keys is None else keys.c()
    p = None if pooled is None else pooled.c()
    vc = None if v is None else v.c()
    _check("indexpool_append", LIB.indexpool_append(
        ctypes.byref(s), kv_new.data_ptr(), ctypes.byref(kc), _ptr(v_new),
        None if vc is None else ctypes.byref(vc), _ptr(key_new),
        _DT[key_new.dtype] if key_new is not None else IP_BF16, None if k is None else ctypes.byref(k),
        _ptr(logit_new), _ptr(logits), None if p is None else ctypes.byref(p), _stream(stream)))


def index_scores_ld(max_seq_len: int) -> int:
    return int(LIB.index_scores_ld(max_seq_len))


def index_score_topk_workspace_bytes(seqs: Seqs, n_q: int, top_k: int, scores_given: bool = False) -> int:
    s = seqs.c()
    return int(LIB.index_score_topk_workspace_bytes(ctypes.byref(s), n_q, top_k, int(scores_given)))


def index_score_topk(seqs: Seqs, q_idx: torch.Tensor, gates: torch.Tensor, pooled: Cache, top_k: int,
                     out_idx: torch.Tensor, q_seq: Optional[torch.Tensor] = None,
                     q_pos: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, stream=None) -> None:
    s, p = seqs.c(), pooled.c()
    n_q, H, D = q_idx.shape
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("index_score_topk", LIB.index_score_topk(
        ctypes.byref(s), n_q, _ptr(q_seq), _ptr(q_pos), q_idx.data_ptr(), _DT[q_idx.dtype], H, D,
        gates.data_ptr(), ctypes.byref(p), top_k, out_idx.data_ptr(), _ptr(scores), _ptr(ws), ws_bytes,
        _stream(stream)))


def index_score_topk_noalloc(seqs: Seqs, q_idx: torch.Tensor, gates: torch.Tensor, pooled: Cache, top_k: int,
                             out_idx: torch.Tensor, q_seq: Optional[torch.Tensor] = None,
                             q_pos: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                             stream=None) -> None:
    s, p = seqs.c(), pooled.c()
    n_q, H, D = q_idx.shape
    _check("index_score_topk_noalloc", LIB.index_score_topk_noalloc(
        ctypes.byref(s), n_q, _ptr(q_seq), _ptr(q_pos), q_idx.data_ptr(), _DT[q_idx.dtype], H, D,
        gates.data_ptr(), ctypes.byref(p), top_k, out_idx.data_ptr(), _ptr(scores), _stream(stream)))


def index_score_topk_noalloc_max_bytes() -> int:
    return int(LIB.index_score_topk_noalloc_max_bytes())


def sparse_attn_workspace_bytes(n_q: int, n_heads: int, dv: int, top_k: int, q_dtype: int) -> int:
    return int(LIB.sparse_attn_workspace_bytes(n_q, n_heads, dv, top_k, q_dtype))


def sparse_attn_decode(seqs: Seqs, q: torch.Tensor, k: Cache, v: Optional[Cache], sel_idx: torch.Tensor,
                       out: torch.Tensor, scale: float, dv: int, lse: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None, stream=None) -> None:
    s, kc = seqs.c(), k.c()
    vc = None if v is None else v.c()
    _, H, dk = q.shape
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("sparse_attn_decode", LIB.sparse_attn_decode(
        ctypes.byref(s), q.data_ptr(), _DT[q.dtype], H, dk, dv, scale, ctypes.byref(kc),
        None if vc is None else ctypes.byref(vc), sel_idx.data_ptr(), sel_idx.shape[1], out.data_ptr(),
        _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def sparse_attn_prefill(seqs: Seqs, q: torch.Tensor, k: Cache, v: Optional[Cache], sel_idx: torch.Tensor,
                        out: torch.Tensor, scale: float, dv: int, q_seq: Optional[torch.Tensor],
                        q_pos: torch.Tensor, lse: Optional[torch.Tensor] = None,
                        ws: Optional[torch.Tensor] = None, stream=None) -> None:
    s, kc = seqs.c(), k.c()
    vc = None if v is None else v.c()
    n_q, H, dk = q.shape
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("sparse_attn_prefill", LIB.sparse_attn_prefill(
        ctypes.byref(s), n_q, _ptr(q_seq), q_pos.data_ptr(), q.data_ptr(), _DT[q.dtype], H, dk, dv, scale,
        ctypes.byref(kc), None if vc is None else ctypes.byref(vc), sel_idx.data_ptr(), sel_idx.shape[1],
        out.data_ptr(), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def time_next_launch(kernel_id: int, start, stop) -> None:
    """The next launch of ``kernel_id`` stores its dispatch start / end times in two
    torch.cuda.Event objects (kernel_id 0 with both None disarms every hook)."""
    a = None if start is None else start.cuda_event
    b = None if stop is None else stop.cuda_event
    _check("ip_time_next_launch", LIB.ip_time_next_launch(kernel_id, a, b))


def version() -> str:
    return LIB.ip_version().decode()


def kda_decode_step(xq: torch.Tensor, xk: torch.Tensor, xv: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                    conv_w: torch.Tensor, conv_in: torch.Tensor, conv_out: torch.Tensor, state: torch.Tensor,
                    out: torch.Tensor, stream=None) -> None:
    """One KDA decode step; state [B, H, 128, 128] is updated in place, the shifted
    conv taps go from conv_in to conv_out."""
    B, H = state.shape[0], state.shape[1]
    _check("kda_decode_step", LIB.kda_decode_step(
        B, H, state.shape[2], xq.data_ptr(), xk.data_ptr(), xv.data_ptr(), _DT[xq.dtype], alpha.data_ptr(),
        beta.data_ptr(), conv_w.data_ptr(), conv_in.data_ptr(), conv_out.data_ptr(), state.data_ptr(),
        out.data_ptr(), _stream(stream)))


def indexpool_decode_index(seqs: Seqs, kv_new: torch.Tensor, kv: Cache, key_new: torch.Tensor, keys: Cache,
                           logit_new: torch.Tensor, logits: torch.Tensor, pooled: Cache, q_idx: torch.Tensor,
                           gates: torch.Tensor, top_k: int, out_idx: torch.Tensor, scores: Optional[torch.Tensor] = None,
                           ws: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
                           v: Optional[Cache] = None, stream=None) -> None:
    """indexpool_append then index_score_topk for the decode rows, in one call."""
    s, kc, k, p = seqs.c(), kv.c(), keys.c(), pooled.c()
    vc = None if v is None else v.c()
    _check("indexpool_decode_index", LIB.indexpool_decode_index(
        ctypes.byref(s), kv_new.data_ptr(), ctypes.byref(kc), _ptr(v_new), None if vc is None else ctypes.byref(vc),
        key_new.data_ptr(), _DT[key_new.dtype], ctypes.byref(k), logit_new.data_ptr(), logits.data_ptr(),
        ctypes.byref(p), q_idx.data_ptr(), _DT[q_idx.dtype], q_idx.shape[1], q_idx.shape[2], gates.data_ptr(),
        top_k, out_idx.data_ptr(), _ptr(scores), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))



def indexpool_decode_step_workspace_bytes(seqs: Seqs, top_k: int, n_heads: int, dv: int, q_dtype: int,
                                          scores_given: bool = False) -> int:
    return int(LIB.indexpool_decode_step_workspace_bytes(ctypes.byref(seqs.c()), top_k, n_heads, dv, q_dtype,
                                                         int(scores_given)))


def indexpool_decode_step(seqs: Seqs, kv_new: torch.Tensor, kv: Cache, key_new: torch.Tensor, keys: Cache,
                          logit_new: torch.Tensor, logits: torch.Tensor, pooled: Cache, q_idx: torch.Tensor,
                          gates: torch.Tensor, top_k: int, out_idx: torch.Tensor, q: torch.Tensor, out: torch.Tensor,
                          scale: float, dv: int, lse: Optional[torch.Tensor] = None,
                          scores: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                          v_new: Optional[torch.Tensor] = None, v: Optional[Cache] = None, stream=None) -> None:
    """indexpool_decode_index then sparse_attn_decode over its selection, in one call."""
    s, kc, k, p = seqs.c(), kv.c(), keys.c(), pooled.c()
    vc = None if v is None else v.c()
    _, H, dk = q.shape
    _check("indexpool_decode_step", LIB.indexpool_decode_step(
        ctypes.byref(s), kv_new.data_ptr(), ctypes.byref(kc), _ptr(v_new), None if vc is None else ctypes.byref(vc),
        key_new.data_ptr(), _DT[key_new.dtype], ctypes.byref(k), logit_new.data_ptr(), logits.data_ptr(),
        ctypes.byref(p), q_idx.data_ptr(), _DT[q_idx.dtype], q_idx.shape[1], q_idx.shape[2], gates.data_ptr(),
        top_k, out_idx.data_ptr(), _ptr(scores), q.data_ptr(), _DT[q.dtype], H, dk, dv, scale, out.data_ptr(),
        _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def kda_prefill_chunk(xq: torch.Tensor, xk: torch.Tensor, xv: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                      conv_w: torch.Tensor, conv_in: torch.Tensor, conv_out: torch.Tensor, state: torch.Tensor,
                      out: torch.Tensor, stream=None) -> None:
    """KDA over a chunk of tokens: x* [B, T, H*128] bf16, alpha [B, T, H, 128], beta [B, T, H];
    state [B, H, 128, 128] updated in place, taps from conv_in to conv_out, out [B, T, H, 128]."""
    B, T = xq.shape[0], xq.shape[1]
    H = state.shape[1]
    _check("kda_prefill_chunk", LIB.kda_prefill_chunk(
        B, T, H, state.shape[2], xq.data_ptr(), xk.data_ptr(), xv.data_ptr(), _DT[xq.dtype], alpha.data_ptr(),
        beta.data_ptr(), conv_w.data_ptr(), conv_in.data_ptr(), conv_out.data_ptr(), state.data_ptr(),
        out.data_ptr(), _stream(stream)))
