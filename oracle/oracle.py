"""CPU oracle for the IndexPool indexer + block-sparse attention path.

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow, float64 restatement of
what the path computes.  Only the tests, the smoke check and the benchmark's CPU
baseline may use it; the library never calls it and shares no code with it.

What it follows (pages are cited by title and section):

* The pipeline: full token history -> MLA latent cache (rank 512 per token) ->
  IndexPool (four indexer keys -> one pooled key) -> learned sparse selection
  (top 2048 tokens) -> attention over the selected history.  G2C Brief
  "GLM-5.3-Flash: hybrid attention becomes the product", section "DSA keeps
  selected global access in eleven layers" (the pipeline figure and the
  ``index_kpool`` / ``index_topk`` / ``kv_lora_rank`` config fields).
* IndexPool: four indexer key vectors merged into one by weighted pooling with
  learned weights instead of QSA's plain mean.  Reading notes "GLM-5.3-Flash:
  Hybrid Attention, IndexPool, and Vision-in-the-Loop", section 2, sub-section
  "IndexPool"; "GLM-5.3-Flash Targets High-Efficiency Inference ...", section
  "Memory and Compute Optimization: IndexPool and KV-Cache Compression".
* The lightweight indexer as the global retriever of the hybrid layer (reading
  notes, section 2 "Hybrid Attention: Linear State + Sparse Retrieval"), in the
  lineage of DeepSeek-V3.2's DSA indexer named there.
* FP8 cache tier (reading notes, section 4 "The serving stack": INT8 / FP8 / BF16
  chosen per cache tier).

Readings taken where the pages are silent (each one is a choice, listed again
in the design notes):

* R1 pooling weights: one logit per cached token; w = softmax of the block's 4
  logits.  A fixed per-position weight vector is the special case of repeated
  logits; equal logits give QSA's plain mean.
* R2 one pooled key per block, shared by all indexer heads.
* R3 pooled fp8 keys are requantised: sigma = max|K| / 448, code = e4m3fn(K/sigma)
  rounded to nearest even, saturating at +-448.  sigma = 0 gives all-zero codes.
* R4 score S_j = sum_h g_h * relu(q_h . K_j), no extra constant.
* R5 selection: the query's own block b_q = floor(p/4) is always kept and counts
  toward k; the other k'-1 = min(k, b_q+1) - 1 are the best-scoring blocks j < b_q
  ordered by (-S_j, j) (ties to the lower index); ids returned ascending, then
  padded with -1.  The own block is never scored.
* R6 attention runs over tokens t = 4j+i of the selected blocks with t <= p;
  logits scale * q.K_t, softmax, weighted sum of V_t; lse = log sum exp.  For the
  576-dim latent row, K is the whole row and V its first 512 dims.
* R7 e4m3fn: bias 7, no infinities, S.1111.111 is NaN, max finite 448.
* R8 decode cache growth: the new token of sequence b sits at t = seq_lens[b] - 1
  (the length already counts it).  Its latent row and logit are stored as given;
  an fp8 key cache stores the key quantised per token like R3 (sigma_t = max|x| /
  448); a float key cache stores the key as given.  When seq_lens[b] % 4 == 0 the
  token completes block t // 4, which is pooled from tokens t-3 .. t (R1-R3).  G2C
  Brief, section "DSA keeps selected global access in eleven layers" (a
  token-addressable history that grows with the sequence); reading notes, section
  4 "The serving stack" (the FP8 tier).
* R9 lower-precision latent tier: the latent row of token t is stored as e4m3fn
  codes with one fp32 scale per token, sigma_t = max|row| / 448 (R3's rule over the
  576 dims), and attention uses sigma_t * dec(code_t) for K and its first 512 dims
  for V.  Reading notes, section 4 "The serving stack" (INT8 / FP8 / BF16 chosen
  per cache tier).
* R10 IndexCache: the DSA layers form groups; the first layer of a group runs the
  indexer (pool, score, select) and every other layer of the group attends, with its
  own queries and latent cache, over that layer's selected blocks, keeping no
  indexer state of its own.  Reading notes, section 2, sub-section "IndexPool" (the
  cross-layer variant of pooling the index is named IndexCache, nothing more).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
E4M3_MAX = 448.0


# ----------------------------------------------------------------------------- fp8
def fp8_decode(codes) -> np.ndarray:
    """e4m3fn code -> value (R7).  Exponent field e, mantissa m, bias 7:
    e > 0: (1 + m/8) * 2^(e-7);  e = 0: (m/8) * 2^-6;  e = 15, m = 7: NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def fp8_encode(x) -> np.ndarray:
    """value -> e4m3fn code, round to nearest even, saturating at +-448 (R3, R7).

    The representable magnitudes in binade [2^e, 2^(e+1)) are spaced 2^(e-3) for
    e >= -6; below 2^-6 the spacing is the subnormal step 2^-9.  The sign of the
    input is kept, so a negative value that rounds to zero gives code 0x80.
    """
    x = np.asarray(x, dtype=F64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, ex = np.frexp(a)                    # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    quantum = np.exp2(e - 3.0)
    v = np.rint(a / quantum) * quantum     # np.rint rounds half to even
    # bits of the rounded magnitude
    fv, ev = np.frexp(v)
    ev = ev.astype(np.int64) - 1           # v = (2 fv) * 2^ev
    sub = v < 2.0 ** -6
    m_sub = np.rint(v / 2.0 ** -9).astype(np.int64)            # 0..7
    biased = ev + 7
    mant = np.rint((2.0 * fv - 1.0) * 8.0).astype(np.int64)
    code = np.where(sub, m_sub, (biased << 3) | mant)
    code = np.where(v == 0, 0, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


# ----------------------------------------------------------------------------- layout
def token_rows(inp, b: int, t) -> np.ndarray:
    """Physical cache row of token t of sequence b (contiguous or paged)."""
    t = np.asarray(t, dtype=np.int64)
    if inp.page_table is None:
        return b * int(inp.seq_stride) + t
    pt = int(inp.page_tokens)
    return inp.page_table[b, t // pt].astype(np.int64) * pt + t % pt


def pooled_rows(inp, b: int, j) -> np.ndarray:
    """Physical pooled row of block j of sequence b.  Blocks never straddle a page,
    so pooled row r always covers token rows 4r .. 4r+3."""
    return token_rows(inp, b, 4 * np.asarray(j, dtype=np.int64)) // 4


# ----------------------------------------------------------------------------- IndexPool
def pool_weights(logits4) -> np.ndarray:
    """R1: w = softmax over the 4 logits of each block (last axis)."""
    l = np.asarray(logits4, dtype=F64)
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def pool_f32(keys4, logits4) -> np.ndarray:
    """Pooled key of each block for float keys: K_hat = sum_i w_i k_i.
    keys4 [N, 4, D], logits4 [N, 4] -> [N, D] float64."""
    w = pool_weights(logits4)
    k = np.asarray(keys4, dtype=F64)
    return (w[:, :, None] * k).sum(axis=1)


def pool_fp8(codes4, scale4, logits4):
    """Pooled fp8 key of each block (R1-R3).

    codes4 [N, 4, D] uint8, scale4 [N, 4], logits4 [N, 4] ->
      codes [N, D] uint8, sigma [N] float64,
      v [N, D] float64 = K_hat / sigma before rounding (0 where sigma = 0),
      mag [N, D] float64 = sum_i |w_i s_i dec(c_i)| / sigma (size of the terms,
      used by tests to bound float32 rounding of the device's sum).
    """
    w = pool_weights(logits4)
    terms = (w * np.asarray(scale4, dtype=F64))[:, :, None] * fp8_decode(codes4)
    k_hat = terms.sum(axis=1)
    sigma = np.abs(k_hat).max(axis=1) / E4M3_MAX
    safe = np.where(sigma > 0, sigma, 1.0)
    v = np.where(sigma[:, None] > 0, k_hat / safe[:, None], 0.0)
    codes = fp8_encode(v)
    codes[sigma == 0] = 0
    mag = np.abs(terms).sum(axis=1) / safe[:, None]
    return codes, sigma, v, mag


def compress(inp):
    """IndexPool over every complete block of every sequence.

    Returns (pooled, sigma, v, mag) indexed by physical pooled row, plus the list
    of valid pooled rows.  fp8 keys: pooled is uint8 codes [R/4, D] and sigma
    float64 [R/4]; float keys: pooled is float64 [R/4, D] and sigma None.
    """
    D = inp.idx_keys.shape[1]
    Rp = inp.idx_keys.shape[0] // 4
    rows = []
    for b in range(len(inp.seq_lens)):
        nb = int(inp.seq_lens[b]) // 4
        rows.append(pooled_rows(inp, b, np.arange(nb)))
    rows = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    tok = (4 * rows[:, None] + np.arange(4)[None, :])
    lg = inp.pool_logits[tok]
    if inp.idx_scale is None:
        pooled = np.zeros((Rp, D), dtype=F64)
        pooled[rows] = pool_f32(inp.idx_keys[tok], lg)
        return pooled, None, None, None, rows
    codes = np.zeros((Rp, D), dtype=np.uint8)
    sigma = np.zeros(Rp, dtype=F64)
    v = np.zeros((Rp, D), dtype=F64)
    mag = np.zeros((Rp, D), dtype=F64)
    step = 1 << 16
    for s0 in range(0, len(rows), step):
        r = rows[s0:s0 + step]
        t = tok[s0:s0 + step]
        c, sg, vv, mg = pool_fp8(inp.idx_keys[t], inp.idx_scale[t], lg[s0:s0 + step])
        codes[r], sigma[r], v[r], mag[r] = c, sg, vv, mg
    return codes, sigma, v, mag, rows


def pooled_values(pooled, sigma) -> np.ndarray:
    """Dequantised pooled keys, float64: sigma_j * dec(code_j) (or the float keys)."""
    if sigma is None:
        return np.asarray(pooled, dtype=F64)
    return np.asarray(sigma, dtype=F64)[:, None] * fp8_decode(pooled)


# ----------------------------------------------------------------------------- decode append
def quantize_tokens(x):
    """Per-token fp8 quantisation of key rows (R8, with R3's rule): sigma =
    max_d |x_d| / 448, codes = e4m3fn(x / sigma), zero codes when sigma = 0.
    x [N, D] -> codes [N, D] uint8, sigma [N] float64, v [N, D] = x / sigma."""
    x = np.asarray(x, dtype=F64)
    sigma = np.abs(x).max(axis=1) / E4M3_MAX
    safe = np.where(sigma > 0, sigma, 1.0)
    v = np.where(sigma[:, None] > 0, x / safe[:, None], 0.0)
    codes = fp8_encode(v)
    codes[sigma == 0] = 0
    return codes, sigma, v


def append(inp, kv_new, key_new, logit_new, only=None):
    """What one decode step's cache growth writes (R8), per sequence.

    inp holds the caches before the step (idx_keys, idx_scale, pool_logits and the
    layout) and seq_lens counting the new tokens.  kv_new [B, ...], key_new [B, D]
    (bf16 bit patterns or floats), logit_new [B].  Returns one dict per sequence with
    a new token: row, kv (for an fp8 latent tier (R9) its codes, with kv_sigma and
    kv_v), key (codes, or floats for a float cache), sigma, v (x / sigma), logit, and when a block completes prow, pooled, psigma, pv, pmag (the
    outputs of pool_fp8, or the float pooled key).  `only`: a subset of sequences
    (the others get None)."""
    out = []
    fp8 = inp.idx_scale is not None
    for b, L in enumerate(np.asarray(inp.seq_lens, dtype=np.int64)):
        if L < 1 or (only is not None and b not in only):
            out.append(None)
            continue
        t = int(L) - 1
        row = int(token_rows(inp, b, t))
        x = _to_f64(np.asarray(key_new)[b])
        e = {"row": row, "kv": np.asarray(kv_new)[b], "logit": float(np.asarray(logit_new)[b])}
        if getattr(inp, "latent_scale", None) is not None:
            # R9: the latent row goes into the fp8 tier quantised per token
            kc, ks, kvv = quantize_tokens(_to_f64(e["kv"])[None])
            e.update(kv=kc[0], kv_sigma=float(ks[0]), kv_v=kvv[0])
        if inp.idx_keys is None:
            # R10: a layer without indexer state keeps only the latent row
            out.append(e)
            continue
        if fp8:
            codes, sigma, v = quantize_tokens(x[None])
            e.update(key=codes[0], sigma=float(sigma[0]), v=v[0])
        else:
            e.update(key=x, sigma=None, v=None)
        if L % 4 == 0:
            prev = token_rows(inp, b, np.arange(t - 3, t))
            lg4 = np.concatenate([np.asarray(inp.pool_logits, dtype=F64)[prev], [e["logit"]]])[None]
            e["prow"] = int(pooled_rows(inp, b, t // 4))
            if fp8:
                c4 = np.concatenate([inp.idx_keys[prev], e["key"][None]])[None]
                s4 = np.concatenate([np.asarray(inp.idx_scale, dtype=F64)[prev], [e["sigma"]]])[None]
                pc, ps, pv, pm = pool_fp8(c4, s4, lg4)
                e.update(pooled=pc[0], psigma=float(ps[0]), pv=pv[0], pmag=pm[0])
            else:
                k4 = np.concatenate([np.asarray(inp.idx_keys, dtype=F64)[prev], x[None]])[None]
                e.update(pooled=pool_f32(k4, lg4)[0], psigma=None, pv=None, pmag=None)
        out.append(e)
    return out


# ----------------------------------------------------------------------------- indexer
def score(q_idx, gates, keys) -> np.ndarray:
    """R4: S_j = sum_h g_h * relu(q_h . K_j).  q_idx [H, D], gates [H], keys [n, D]."""
    dots = np.asarray(keys, dtype=F64) @ np.asarray(q_idx, dtype=F64).T   # [n, H]
    return np.maximum(dots, 0.0) @ np.asarray(gates, dtype=F64)


def score_many(q_idx, gates, keys) -> np.ndarray:
    """R4 for several query rows over one key set: S[r, j] = sum_h g[r, h] *
    relu(q[r, h] . K_j).  q_idx [R, H, D], gates [R, H], keys [n, D] -> [R, n]."""
    q = np.asarray(q_idx, dtype=F64)
    R, H, D = q.shape
    dots = np.asarray(keys, dtype=F64) @ q.reshape(R * H, D).T            # [n, R*H]
    dots = np.maximum(dots, 0.0).reshape(-1, R, H)
    return np.einsum("nrh,rh->rn", dots, np.asarray(gates, dtype=F64))


def select(S, b_q: int, k: int) -> np.ndarray:
    """R5: own block plus the best k'-1 blocks j < b_q; ascending; -1 padded to k."""
    S = np.asarray(S, dtype=F64)[:b_q]
    kp = min(k, b_q + 1)
    j = np.arange(b_q)
    order = np.lexsort((j, -S))            # primary -S, then j
    chosen = np.sort(order[: kp - 1])
    out = np.full(k, -1, dtype=np.int32)
    out[: kp - 1] = chosen
    out[kp - 1] = b_q
    return out


def row_scores(inp, pooled_vals, r: int) -> np.ndarray:
    """Scores of query row r over its eligible blocks j < b_q."""
    b = int(inp.q_seq[r])
    b_q = int(inp.q_pos[r]) // 4
    keys = pooled_vals[pooled_rows(inp, b, np.arange(b_q))]
    return score(_to_f64(inp.q_idx[r]), inp.gates[r], keys)


def score_select(inp, pooled_vals, k: int, rows=None):
    """Selected block ids [len(rows), k] and the per-row score vectors."""
    rows = range(len(inp.q_pos)) if rows is None else rows
    ids, scores = [], []
    for r in rows:
        S = row_scores(inp, pooled_vals, r)
        scores.append(S)
        ids.append(select(S, int(inp.q_pos[r]) // 4, k))
    return np.stack(ids), scores


# ----------------------------------------------------------------------------- attention
def attend(q, K, V, scale: float):
    """R6 over one token set: q [H, dk], K [n, dk], V [n, dv] -> O [H, dv], lse [H]."""
    logits = scale * (np.asarray(q, dtype=F64) @ np.asarray(K, dtype=F64).T)   # [H, n]
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    l = e.sum(axis=1, keepdims=True)
    O = (e @ np.asarray(V, dtype=F64)) / l
    return O, (m + np.log(l))[:, 0]


def selected_tokens(ids, pos: int) -> np.ndarray:
    """Tokens 4j+i of the selected blocks (ids >= 0) with 4j+i <= pos, ascending."""
    j = np.asarray(ids, dtype=np.int64)
    j = j[j >= 0]
    t = (4 * j[:, None] + np.arange(4)[None, :]).reshape(-1)
    return t[t <= pos]


def _to_f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:     # bf16 bit patterns
        return (x.astype(np.uint32) << 16).view(np.float32).astype(F64)
    return x.astype(F64)


def latent_rows(inp, phys) -> np.ndarray:
    """Latent rows as float64: bf16 rows widened, or (R9) the fp8 tier's
    sigma_t * dec(code_t) with one scale per token row."""
    if getattr(inp, "latent_scale", None) is not None:
        return np.asarray(inp.latent_scale, dtype=F64)[phys][:, None] * fp8_decode(inp.latent[phys])
    return _to_f64(inp.latent[phys])


def attention_rows(inp, ids, scale: float, dv: int, rows=None):
    """Sparse attention for query rows (default all): O [n, H, dv], lse [n, H]."""
    rows = range(len(inp.q_pos)) if rows is None else rows
    outs, lses = [], []
    for n, r in enumerate(rows):
        b = int(inp.q_seq[r])
        t = selected_tokens(ids[n], int(inp.q_pos[r]))
        phys = token_rows(inp, b, t)
        if inp.latent is not None:
            KV = latent_rows(inp, phys)
            K, V = KV, KV[:, :dv]
        else:
            K = _to_f64(inp.k_cache[phys])
            V = _to_f64(inp.v_cache[phys])
        O, lse = attend(_to_f64(inp.q[r]), K, V, scale)
        outs.append(O)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


# ----------------------------------------------------------------------------- IndexCache
def indexcache_group(anchor, followers, scale: float, dv: int, top_k: int, rows=None):
    """R10: the first layer (`anchor`) selects; it and every follower layer attend over
    that one selection.  Returns the anchor's ids [n, top_k] and one (O, lse) per layer,
    anchor first."""
    pooled, sigma, *_ = compress(anchor)
    ids, _ = score_select(anchor, pooled_values(pooled, sigma), top_k, rows=rows)
    outs = [attention_rows(x, ids, scale, dv, rows=rows) for x in [anchor, *followers]]
    return ids, outs

