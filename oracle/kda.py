"""CPU oracle for the KDA (linear-attention) decode step of the hybrid layer.

TEST INFRASTRUCTURE ONLY.  A plain, slow, float64 restatement of one recurrent
step; only the tests, the smoke check and the benchmark's CPU baseline may use it.
It shares no code with the library.

What the pages fix (cited by title and section):

* G2C Brief "GLM-5.3-Flash: hybrid attention becomes the product", section "KDA
  carries fixed state through most layers": 34 of the 45 layers are Kimi Delta
  Attention, a linear-attention variant built on the gated delta rule, which keeps
  one fixed-size matrix per head in place of a cached row per token; a short
  convolution (``short_conv_kernel_size: 4``) and learned gates surround it.
* The same brief, release summary: 64 heads of width 128, so the state is a
  128 x 128 matrix per head (64 x 128 x 128 values per layer), independent of the
  context length.
* Reading notes, section 2 "Hybrid Attention: Linear State + Sparse Retrieval":
  the linear half costs the same per token at any context length.

Readings taken where the pages are silent (listed again in the design notes):

* K1 per-head recurrence, the gated delta rule with a per-channel decay (the
  fine-grained gate of Kimi Delta Attention as published):
      S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
      o_t = S_t^T q_t / sqrt(d_k)
  with S [d_k, d_v] (rows = key channels), alpha_t in (0, 1]^d_k the decay of each
  key channel and beta_t in (0, 1) the write strength, both given per token and
  head (their projections belong to the model and are inputs here).
* K2 short convolution: q, k and v each pass a causal depthwise convolution of
  width 4 over time (taps x_{t-3} .. x_t, one weight vector per channel), then
  SiLU.  The step keeps the last 3 inputs per channel as conv state.
* K3 q and k are L2-normalised per head after the convolution (eps 1e-6 under the
  square root), the usual stabiliser of delta-rule recurrences.
* K4 precision: the state and the conv state are fp32 in memory; inputs x_q, x_k,
  x_v are bf16, alpha, beta and the conv weights fp32; the output is fp32.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
CONV = 4          # K2: short_conv_kernel_size
EPS = 1e-6        # K3


def silu(x):
    x = np.asarray(x, dtype=F64)
    return x / (1.0 + np.exp(-x))


def short_conv(hist, x, w):
    """K2 for one token: hist [3, C] holds x_{t-3}, x_{t-2}, x_{t-1}; x [C] is x_t;
    w [C, 4] the taps (w[:, 3] weighs x_t).  Returns (silu(conv) [C], new hist)."""
    taps = np.concatenate([np.asarray(hist, dtype=F64), np.asarray(x, dtype=F64)[None]])   # [4, C]
    y = (taps.T * np.asarray(w, dtype=F64)).sum(axis=1)
    return silu(y), taps[1:]


def l2norm(x):
    """K3 over the last axis."""
    x = np.asarray(x, dtype=F64)
    return x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + EPS)


def delta_step(S, q, k, v, alpha, beta):
    """K1 for one head: S [dk, dv], q, k [dk], v [dv], alpha [dk], beta scalar.
    Decay the key channels, then write v at k with the delta rule, then read at q."""
    S = np.asarray(S, dtype=F64)
    k = np.asarray(k, dtype=F64)
    Sd = np.asarray(alpha, dtype=F64)[:, None] * S           # Diag(alpha) S
    u = Sd.T @ k                                             # what the state returns for k
    S_new = Sd + beta * np.outer(k, np.asarray(v, dtype=F64) - u)
    o = S_new.T @ np.asarray(q, dtype=F64) / np.sqrt(S.shape[0])
    return S_new, o


def decode_step(state, conv_state, xq, xk, xv, alpha, beta, conv_w):
    """One KDA decode step for a batch.

    state [B, H, dk, dv]; conv_state [B, 3 (q, k, v), 3 (taps t-3..t-1), H*d];
    xq, xk [B, H*dk], xv [B, H*dv] (any float dtype, bf16 given as float32 values);
    alpha [B, H, dk]; beta [B, H]; conv_w [3, H*d, 4].
    Returns (new state, new conv state, o [B, H, dv])."""
    state = np.asarray(state, dtype=F64)
    B, H, dk, dv = state.shape
    S_out = np.empty_like(state)
    cs_out = np.empty(np.shape(conv_state), dtype=F64)
    o = np.empty((B, H, dv))
    for b in range(B):
        yq, cs_out[b, 0] = short_conv(conv_state[b][0], xq[b], conv_w[0])
        yk, cs_out[b, 1] = short_conv(conv_state[b][1], xk[b], conv_w[1])
        yv, cs_out[b, 2] = short_conv(conv_state[b][2], xv[b], conv_w[2])
        q = l2norm(yq.reshape(H, dk))
        k = l2norm(yk.reshape(H, dk))
        v = yv.reshape(H, dv)
        for h in range(H):
            S_out[b, h], o[b, h] = delta_step(state[b, h], q[h], k[h], v[h], alpha[b, h], float(beta[b, h]))
    return S_out, cs_out, o


def prefill_chunk(state, conv_state, xq, xk, xv, alpha, beta, conv_w):
    """The reference of the chunked (prefill) form: the recurrence of decode_step run
    token by token over a chunk of T tokens.  xq, xk [B, T, H*dk], xv [B, T, H*dv]
    (float values), alpha [B, T, H, dk], beta [B, T, H]; state and conv_state as for
    decode_step.  Returns (state, conv state, o [B, T, H, dv])."""
    S, cs = np.asarray(state, dtype=F64), np.asarray(conv_state, dtype=F64)
    T = np.shape(xq)[1]
    outs = []
    for t in range(T):
        S, cs, o = decode_step(S, cs, xq[:, t], xk[:, t], xv[:, t], alpha[:, t], beta[:, t], conv_w)
        outs.append(o)
    B, H, _, dv = S.shape
    return S, cs, (np.stack(outs, axis=1) if outs else np.zeros((B, 0, H, dv)))
