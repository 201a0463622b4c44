"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test checks the oracle against a library routine, a closed form, a worked
example derived by hand, an invariant the pages state, or brute force on tiny
inputs, so that a dropped term, a wrong sign or index, or a transposed operand
anywhere in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- fp8 codec
def test_fp8_decode_exhaustive_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_fp8_encode_roundtrips_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.fp8_decode(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(O.fp8_encode(vals[fin]), codes[fin])


@pytest.mark.parametrize("scale", [448.0, 1.0, 2.0 ** -6, 2.0 ** -9])
def test_fp8_encode_matches_torch_rne(scale):
    # float32-exact inputs: torch narrows float64 to float32 before the fp8 cast,
    # which would round twice
    x = (np.random.default_rng(7).uniform(-1, 1, 200000) * scale).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.fp8_encode(x), ref)


def test_fp8_encode_midpoints_round_to_even():
    vals = O.fp8_decode(np.arange(0, 0x7E, dtype=np.uint8))   # 0 .. 416 ascending
    mids = (vals[:-1] + vals[1:]) / 2.0
    got = O.fp8_encode(mids)
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    assert np.all(got % 2 == 0)            # even mantissa wins every tie


def test_fp8_encode_saturates_and_flushes():
    assert O.fp8_encode(np.array([464.0, 500.0, 1e9, -1e9])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    assert O.fp8_encode(np.array([2.0 ** -10, 3 * 2.0 ** -11, -2.0 ** -11])).tolist() == [0, 1, 0x80]


# --------------------------------------------------------------------------- IndexPool
def test_pool_worked_example():
    g = _golden("pool_worked_example.json")
    keys = np.array(g["keys"])[None]
    logits = np.array(g["logits"])[None]
    np.testing.assert_allclose(O.pool_f32(keys, logits)[0], g["pooled"], rtol=1e-15)
    # fp8 version: store each key as codes with scale 1 (all values are exact in fp8)
    codes = O.fp8_encode(keys)
    c, sigma, v, _ = O.pool_fp8(codes, np.ones((1, 4)), logits)
    assert c[0].tolist() == g["codes"]
    assert sigma[0] == pytest.approx(g["sigma"], rel=1e-15)


def test_pool_equal_logits_is_plain_mean():
    """QSA's r=4 average-pooled key block is IndexPool with equal weights."""
    rng = np.random.default_rng(1)
    keys = rng.standard_normal((50, 4, 32))
    logits = np.repeat(rng.standard_normal((50, 1)), 4, axis=1)
    np.testing.assert_allclose(O.pool_f32(keys, logits), keys.mean(axis=1), rtol=1e-13, atol=1e-15)
    codes = O.fp8_encode(keys * 100)
    scale = rng.uniform(0.5, 2.0, (50, 4))
    _, sigma, v, _ = O.pool_fp8(codes, scale, logits)
    mean = (scale[:, :, None] * O.fp8_decode(codes)).mean(axis=1)
    np.testing.assert_allclose(v * sigma[:, None], mean, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("hot", [0, 1, 2, 3])
def test_pool_one_hot_logit_copies_that_key(hot):
    """A dominant logit makes the pooled key an exact copy of that token's key;
    for an fp8 row whose max element is coded 448, the requantised codes and
    scale equal the source codes and scale."""
    rng = np.random.default_rng(hot)
    x = rng.standard_normal((20, 4, 64))
    s = np.abs(x).max(axis=2) / 448.0
    codes = O.fp8_encode(x / s[:, :, None])
    logits = np.zeros((20, 4))
    logits[:, hot] = 60.0
    c, sigma, _, _ = O.pool_fp8(codes, s, logits)
    assert np.array_equal(c, codes[:, hot])
    np.testing.assert_allclose(sigma, s[:, hot], rtol=1e-15)
    kf = O.pool_f32(x, logits)
    np.testing.assert_allclose(kf, x[:, hot], rtol=1e-12, atol=1e-12)


def test_pool_identical_keys_give_that_key():
    """Weights sum to one, whatever the logits."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((30, 1, 16))
    keys = np.repeat(k, 4, axis=1)
    logits = rng.standard_normal((30, 4)) * 5
    np.testing.assert_allclose(O.pool_f32(keys, logits), k[:, 0], rtol=1e-13, atol=1e-14)


def test_pool_max_element_codes_448_and_zero_block():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 0x7E, (40, 4, 128), dtype=np.uint8)
    codes[0] = 0                                   # an all-zero block
    scale = rng.uniform(0.01, 1.0, (40, 4))
    c, sigma, v, _ = O.pool_fp8(codes, scale, rng.standard_normal((40, 4)))
    assert sigma[0] == 0 and not c[0].any()
    dec = O.fp8_decode(c[1:])
    assert np.all(np.abs(dec).max(axis=1) == 448.0)


def test_pooled_cache_is_four_times_smaller():
    """The resident indexer state drops 4x: T/4 pooled rows of the same width."""
    from long_context_sparse_19_amd.configs import TINY, DECODE, scaled_down
    from long_context_sparse_19_amd.inputs import make_inputs
    for w in (TINY, scaled_down(DECODE, 4096, batch=2)):
        inp = make_inputs(w, with_attention=False)
        pooled, sigma, *_ , rows = O.compress(inp)
        T = int(inp.seq_lens.sum())
        assert len(rows) == T // 4
        tok_bytes = inp.idx_keys[:T].nbytes + (0 if inp.idx_scale is None else inp.idx_scale[:T].nbytes)
        item = pooled.dtype.itemsize if sigma is not None else 4   # f32 keys stay f32
        pool_bytes = len(rows) * pooled.shape[1] * item + (0 if sigma is None else 4 * len(rows))
        assert tok_bytes == 4 * pool_bytes


# --------------------------------------------------------------------------- scoring
def test_score_select_worked_example():
    g = _golden("score_select_worked_example.json")
    S = O.score(np.array(g["q_idx"]), np.array(g["gates"]), np.array(g["keys"][:5]))
    assert S.tolist() == g["scores"]
    b_q = g["pos"] // 4
    assert O.select(S, b_q, 3).tolist() == g["select_k3"]
    assert O.select(S, b_q, 8).tolist() == g["select_k8"]


def test_score_many_is_score_per_row_and_the_closed_form():
    """score_many (several rows at once) equals the per-row score on random rows,
    and the unit-query closed form row by row."""
    rng = np.random.default_rng(9)
    q = rng.standard_normal((5, 3, 16))
    g = rng.standard_normal((5, 3))
    keys = rng.standard_normal((40, 16))
    S = O.score_many(q, g, keys)
    for r in range(5):
        np.testing.assert_allclose(S[r], O.score(q[r], g[r], keys), rtol=1e-13, atol=1e-13)
    unit = np.zeros((2, 1, 16))
    unit[0, 0, 4] = 1.0
    unit[1, 0, 11] = 1.0
    S = O.score_many(unit, np.ones((2, 1)), keys)
    assert np.array_equal(S[0], np.maximum(keys[:, 4], 0.0))
    assert np.array_equal(S[1], np.maximum(keys[:, 11], 0.0))


def test_score_unit_query_is_relu_of_one_coordinate():
    rng = np.random.default_rng(5)
    keys = rng.standard_normal((100, 24))
    for d in (0, 7, 23):
        q = np.zeros((1, 24))
        q[0, d] = 1.0
        np.testing.assert_array_equal(O.score(q, [1.0], keys), np.maximum(keys[:, d], 0))


def test_score_gates_pick_heads_and_sign():
    rng = np.random.default_rng(6)
    keys = rng.standard_normal((64, 8))
    q = rng.standard_normal((2, 8))
    h0 = np.maximum(keys @ q[0], 0)
    h1 = np.maximum(keys @ q[1], 0)
    np.testing.assert_allclose(O.score(q, [1.0, 0.0], keys), h0, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(O.score(q, [0.0, 1.0], keys), h1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(O.score(q, [-2.0, 0.5], keys), -2 * h0 + 0.5 * h1, rtol=1e-13, atol=1e-13)


def test_score_fp8_pooled_includes_sigma():
    codes = np.array([[0x7E, 0xFE, 0x38]], dtype=np.uint8)   # 448, -448, 1.0
    sigma = np.array([0.25])
    vals = O.pooled_values(codes, sigma)
    assert vals.tolist() == [[112.0, -112.0, 0.25]]
    q = np.eye(3)
    assert O.score(q[[0]], [1.0], vals).tolist() == [112.0]
    assert O.score(q[[1]], [1.0], vals).tolist() == [0.0]
    assert O.score(q[[2]], [1.0], vals).tolist() == [0.25]


# --------------------------------------------------------------------------- selection
def _brute_select(S, b_q, k):
    """j is kept iff fewer than k'-1 blocks beat it under (higher score, lower index)."""
    kp = min(k, b_q + 1)
    keep = []
    for j in range(b_q):
        better = sum(1 for i in range(b_q) if S[i] > S[j] or (S[i] == S[j] and i < j))
        if better < kp - 1:
            keep.append(j)
    return keep + [b_q] + [-1] * (k - kp)


@pytest.mark.parametrize("seed", range(12))
def test_select_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    b_q = int(rng.integers(0, 40))
    k = int(rng.integers(1, 50))
    S = np.round(rng.standard_normal(b_q) * 2) / 2      # many exact ties
    assert O.select(S, b_q, k).tolist() == _brute_select(S, b_q, k)


def test_select_all_when_k_exceeds_blocks_and_own_block_only():
    assert O.select(np.zeros(5), 5, 9).tolist() == [0, 1, 2, 3, 4, 5, -1, -1, -1]
    assert O.select(np.zeros(0), 0, 4).tolist() == [0, -1, -1, -1]
    assert O.select(np.arange(10.0), 10, 1).tolist() == [10]
    # all-equal scores: lowest indices win
    assert O.select(np.zeros(10), 10, 4).tolist() == [0, 1, 2, 10]


# --------------------------------------------------------------------------- attention
def _sdpa_causal(q, K, V, scale, pos):
    """torch scaled_dot_product_attention in float64 with an explicit causal mask."""
    qt = torch.from_numpy(q)[None]                   # [1, n, H, d] -> [1, H, n, d]
    qt = qt.permute(0, 2, 1, 3)
    Kt = torch.from_numpy(K)[None, None].expand(1, q.shape[1], -1, -1)
    Vt = torch.from_numpy(V)[None, None].expand(1, q.shape[1], -1, -1)
    t = torch.arange(K.shape[0])
    mask = t[None, :] <= torch.from_numpy(pos)[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, Kt, Vt, attn_mask=mask[None, None], scale=scale)
    return o.permute(0, 2, 1, 3)[0].numpy()


def test_attend_selecting_every_block_is_dense_causal_attention():
    """With k >= b_q + 1 every earlier block is selected, and the masked own block
    completes the causal prefix: sparse attention equals dense causal attention."""
    rng = np.random.default_rng(8)
    T, H, dk, dv = 64, 3, 16, 8
    K = rng.standard_normal((T, dk))
    V = rng.standard_normal((T, dv))
    pos = np.arange(40, 64)                          # positions inside blocks too
    q = rng.standard_normal((len(pos), H, dk))
    ref = _sdpa_causal(q, K, V, 0.3, pos)
    for n, p in enumerate(pos):
        ids = O.select(np.zeros(p // 4), p // 4, 100)
        t = O.selected_tokens(ids, int(p))
        assert t.tolist() == list(range(p + 1))
        Ot, _ = O.attend(q[n], K[t], V[t], 0.3)
        np.testing.assert_allclose(Ot, ref[n], rtol=1e-12, atol=1e-12)


def test_attend_special_cases():
    rng = np.random.default_rng(9)
    K = rng.standard_normal((12, 6))
    V = rng.standard_normal((12, 5))
    q = rng.standard_normal((4, 6))
    O1, lse1 = O.attend(q, K[3:4], V[3:4], 0.7)          # a single token
    np.testing.assert_array_equal(O1, np.repeat(V[3:4], 4, axis=0))
    np.testing.assert_allclose(lse1, 0.7 * q @ K[3], rtol=1e-14)
    O0, lse0 = O.attend(np.zeros((2, 6)), K, V, 0.7)      # q = 0: plain mean
    np.testing.assert_allclose(O0, np.repeat(V.mean(0, keepdims=True), 2, 0), rtol=1e-13)
    np.testing.assert_allclose(lse0, math.log(12), rtol=1e-14)
    Oa, lse = O.attend(q, K, V, 0.7)
    assert np.all(Oa >= V.min(0) - 1e-12) and np.all(Oa <= V.max(0) + 1e-12)
    ref = np.log(np.exp(0.7 * q @ K.T).sum(1))
    np.testing.assert_allclose(lse, ref, rtol=1e-13)


def test_selected_tokens_causal_inside_own_block():
    ids = np.array([1, 3, 7, -1])
    assert O.selected_tokens(ids, 29).tolist() == [4, 5, 6, 7, 12, 13, 14, 15, 28, 29]


# --------------------------------------------------------------------------- layout
def test_paged_and_contiguous_layouts_agree():
    """A shuffled page table changes only where rows live, never the result."""
    from long_context_sparse_19_amd.configs import RAGGED, scaled_down
    from long_context_sparse_19_amd.inputs import make_inputs
    w = scaled_down(RAGGED, 2048, batch=3, min_blocks=100, top_k=32)
    inp = make_inputs(w)

    class Flat:
        pass
    flat = Flat()
    L = int(inp.seq_lens.max())
    flat.page_table, flat.page_tokens, flat.seq_stride = None, 0, L
    flat.seq_lens, flat.q_seq, flat.q_pos = inp.seq_lens, inp.q_seq, inp.q_pos
    flat.q, flat.q_idx, flat.gates = inp.q, inp.q_idx, inp.gates
    n = len(inp.seq_lens) * L
    flat.idx_keys = np.zeros((n, inp.idx_keys.shape[1]), inp.idx_keys.dtype)
    flat.idx_scale = np.ones(n, np.float32)
    flat.pool_logits = np.zeros(n, np.float32)
    flat.latent = np.zeros((n, inp.latent.shape[1]), np.uint16)
    flat.k_cache = flat.v_cache = None
    for b in range(len(inp.seq_lens)):
        t = np.arange(int(inp.seq_lens[b]))
        src = O.token_rows(inp, b, t)
        dst = b * L + t
        flat.idx_keys[dst] = inp.idx_keys[src]
        flat.idx_scale[dst] = inp.idx_scale[src]
        flat.pool_logits[dst] = inp.pool_logits[src]
        flat.latent[dst] = inp.latent[src]
    outs = []
    for x in (inp, flat):
        pooled, sigma, *_ = O.compress(x)
        vals = O.pooled_values(pooled, sigma)
        ids, _ = O.score_select(x, vals, w.top_k)
        Ox, lse = O.attention_rows(x, ids, w.scale, w.dv)
        outs.append((ids, Ox, lse))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[0][2], outs[1][2])


def test_paged_row_mapping_worked_example():
    """token_rows / pooled_rows against rows worked by hand for a shuffled 8-token
    page table over three sequences, and for a contiguous cache."""
    from types import SimpleNamespace
    g = _golden("paged_rows_worked_example.json")
    pg = g["paged"]
    inp = SimpleNamespace(page_table=np.array(pg["page_table"], dtype=np.int32), page_tokens=pg["page_tokens"],
                          seq_stride=0)
    for b, t, row in pg["token_rows"]:
        assert int(O.token_rows(inp, b, t)) == row, (b, t)
    for b, j, row in pg["pooled_rows"]:
        assert int(O.pooled_rows(inp, b, j)) == row, (b, j)
        # the pooled row covers the token rows of its block's four tokens
        assert (O.token_rows(inp, b, 4 * j + np.arange(4)) // 4 == row).all()
    # vectorised calls give the same rows as the scalar ones
    b, t, rows = zip(*[x for x in pg["token_rows"] if x[0] == 2])
    assert O.token_rows(inp, 2, np.array(t)).tolist() == list(rows)
    ct = g["contiguous"]
    flat = SimpleNamespace(page_table=None, page_tokens=0, seq_stride=ct["seq_stride"])
    for b, t, row in ct["token_rows"]:
        assert int(O.token_rows(flat, b, t)) == row, (b, t)
    for b, j, row in ct["pooled_rows"]:
        assert int(O.pooled_rows(flat, b, j)) == row, (b, j)


def test_score_select_rows_worked_example():
    """Per-row wiring of score_select (sequence of each row, eligible blocks j < b_q,
    the own block kept, k < b_q and k > b_q) against ids and scores worked by hand
    for three prefill rows over two sequences."""
    from types import SimpleNamespace
    g = _golden("score_select_rows_worked_example.json")
    inp = SimpleNamespace(page_table=None, page_tokens=0, seq_stride=g["seq_stride"],
                          seq_lens=np.array(g["seq_lens"], dtype=np.int32),
                          q_seq=np.array(g["q_seq"], dtype=np.int32), q_pos=np.array(g["q_pos"], dtype=np.int32),
                          q_idx=np.array(g["q_idx"]), gates=np.array(g["gates"]))
    ids, scores = O.score_select(inp, np.array(g["pooled"]), g["top_k"])
    assert ids.tolist() == g["ids"]
    assert [s.tolist() for s in scores] == g["scores"]
    # one row at a time through row_scores gives the same scores
    for r in range(len(g["q_pos"])):
        assert O.row_scores(inp, np.array(g["pooled"]), r).tolist() == g["scores"][r]


def test_end_to_end_all_blocks_equals_dense_causal():
    """pool -> score -> select (k covering every block) -> attend reproduces dense
    causal attention over the whole history, for a prefill chunk."""
    from long_context_sparse_19_amd.configs import PREFILL, scaled_down
    from long_context_sparse_19_amd.inputs import make_inputs, bf16_bits_to_f32
    w = scaled_down(PREFILL, 256, n_query=24, top_k=64)
    inp = make_inputs(w)
    pooled, sigma, *_ = O.compress(inp)
    ids, _ = O.score_select(inp, O.pooled_values(pooled, sigma), w.top_k)
    Os, _ = O.attention_rows(inp, ids, w.scale, w.dv)
    KV = bf16_bits_to_f32(inp.latent).astype(np.float64)
    q = bf16_bits_to_f32(inp.q).astype(np.float64)
    ref = _sdpa_causal(q, KV, KV[:, : w.dv].copy(), w.scale, inp.q_pos.astype(np.int64))
    np.testing.assert_allclose(Os, ref, rtol=1e-11, atol=1e-11)


def test_fp8_latent_attention_is_dense_attention_over_dequantised_rows():
    """The fp8 latent tier (R9): with every block selected, sparse attention over
    codes and per-token scales equals dense causal attention (torch) over
    sigma_t * code_t, the codes widened by torch's own e4m3fn cast."""
    from long_context_sparse_19_amd.configs import DECODE_FP8KV, PREFILL, scaled_down
    from long_context_sparse_19_amd.inputs import make_inputs, bf16_bits_to_f32
    for w in (scaled_down(DECODE_FP8KV, 192, batch=2, top_k=64),
              scaled_down(PREFILL.with_(latent_fp8=True), 192, n_query=12, top_k=64)):
        inp = make_inputs(w)
        assert inp.latent.dtype == np.uint8 and inp.latent_scale.dtype == np.float32
        pooled, sigma, *_ = O.compress(inp)
        ids, _ = O.score_select(inp, O.pooled_values(pooled, sigma), w.top_k)
        Os, lse = O.attention_rows(inp, ids, w.scale, w.dv)
        q = bf16_bits_to_f32(inp.q).astype(np.float64)
        for b in range(len(inp.seq_lens)):
            rows = np.flatnonzero(inp.q_seq == b) if w.mode == "prefill" else np.array([b])
            t = np.arange(int(inp.seq_lens[b]))
            phys = O.token_rows(inp, b, t)
            dec = torch.from_numpy(inp.latent[phys]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
            KV = inp.latent_scale[phys].astype(np.float64)[:, None] * dec
            pos = inp.q_pos[rows].astype(np.int64) if w.mode == "prefill" else np.array([t[-1]])
            ref = _sdpa_causal(q[rows], KV, KV[:, : w.dv].copy(), w.scale, pos)
            np.testing.assert_allclose(Os[rows], ref, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------- decode append
def test_quantize_token_closed_form():
    c = 0.37
    x = np.zeros((2, 128))
    x[0, :4] = [448 * c, -224 * c, 1.5 * c, -0.0]
    codes, sigma, v = O.quantize_tokens(x)
    assert sigma[0] == pytest.approx(c, rel=1e-15) and sigma[1] == 0.0
    assert list(codes[0, :3]) == [0x7E, 0xF6, 0x3C]      # +448, -224, +1.5
    assert codes[0, 3] == 0x80 and not codes[0, 4:].any()   # -0.0 keeps its sign
    assert not codes[1].any()


def test_quantize_token_matches_torch_and_error_bound():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 128))
    x[::7] *= 8.0                                     # some larger rows
    codes, sigma, v = O.quantize_tokens(x)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # away from rounding midpoints the float32 cast in torch cannot change the code
    val = O.fp8_decode(codes)
    near_tie = np.zeros_like(v, dtype=bool)
    for delta in (1, -1):
        other = O.fp8_decode(np.clip(codes.astype(np.int64) + delta, 0, 255).astype(np.uint8))
        near_tie |= np.abs(np.abs(v) - (np.abs(val) + np.abs(other)) / 2) <= 1e-6 * np.abs(v)
    assert np.array_equal(codes[~near_tie], ref[~near_tie])
    err = np.abs(sigma[:, None] * val - x)
    bound = np.maximum(2.0 ** -4 * np.abs(x), sigma[:, None] * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-12))
    assert np.all(np.abs(val).max(axis=1) == 448.0)


def _append_state(fp8, paged=False, seed=5):
    """A small cache (3 sequences of up to 16 tokens) and new tokens for append."""
    from types import SimpleNamespace
    rng = np.random.default_rng(seed)
    B, S, D = 3, 16, 128 if fp8 else 8
    lens = np.array([8, 7, 13], dtype=np.int32)
    if fp8:
        keys, scale = O.quantize_tokens(rng.standard_normal((B * S, D)))[:2]
    else:
        keys, scale = rng.standard_normal((B * S, D)), None
    st = SimpleNamespace(idx_keys=keys, idx_scale=scale, pool_logits=rng.standard_normal(B * S),
                         seq_lens=lens, page_table=None, seq_stride=S, page_tokens=0)
    if paged:
        perm = rng.permutation(B * S // 8).reshape(B, S // 8)     # 8-token pages, shuffled
        st.page_table, st.page_tokens = perm.astype(np.int32), 8
    new = dict(kv_new=rng.standard_normal((B, 576)), key_new=rng.standard_normal((B, D)),
               logit_new=rng.standard_normal(B))
    return st, new


@pytest.mark.parametrize("fp8", [True, False])
@pytest.mark.parametrize("paged", [False, True])
def test_append_writes_the_new_token_and_pools_completed_blocks(fp8, paged):
    """Growth then pooling agree with a cache build: writing the new token into the
    cache and running compress over it gives the pooled block that append reports;
    only a length that is a multiple of 4 pools, and the token goes to row L - 1."""
    st, new = _append_state(fp8, paged)
    res = O.append(st, **new)
    for b, e in enumerate(res):
        L = int(st.seq_lens[b])
        assert e["row"] == int(O.token_rows(st, b, L - 1))
        assert ("prow" in e) == (L % 4 == 0)
        assert e["logit"] == new["logit_new"][b]
        if fp8:
            c, s, _ = O.quantize_tokens(new["key_new"][b][None])
            assert np.array_equal(e["key"], c[0]) and e["sigma"] == s[0]
    # the cache after the step, pooled by the cache build
    grown = type(st)(**vars(st))
    grown.idx_keys = st.idx_keys.copy()
    grown.pool_logits = st.pool_logits.copy()
    if fp8:
        grown.idx_scale = st.idx_scale.copy()
    for e in res:
        grown.idx_keys[e["row"]] = e["key"]
        grown.pool_logits[e["row"]] = e["logit"]
        if fp8:
            grown.idx_scale[e["row"]] = e["sigma"]
    pooled, sigma, *_ = O.compress(grown)
    e = res[0]                                        # L = 8 completes block 1
    assert e["prow"] == int(O.pooled_rows(st, 0, 1))
    if fp8:
        assert np.array_equal(pooled[e["prow"]], e["pooled"]) and sigma[e["prow"]] == e["psigma"]
    else:
        np.testing.assert_allclose(pooled[e["prow"]], e["pooled"], rtol=1e-15, atol=0)


def test_append_quantises_the_latent_row_for_the_fp8_tier():
    """R9 with R8: the new latent row enters the fp8 tier as torch's e4m3fn cast of
    row / sigma (sigma = max|row| / 448), within half a code step of the row."""
    from long_context_sparse_19_amd.configs import DECODE_FP8KV, scaled_down
    from long_context_sparse_19_amd.inputs import make_inputs, new_tokens, bf16_bits_to_f32
    w = scaled_down(DECODE_FP8KV, 64, batch=3, top_k=8)
    inp = make_inputs(w)
    new = new_tokens(w, 3, seed=5)
    res = O.append(inp, new["kv_new"], new["key_new"], new["logit_new"])
    for b, e in enumerate(res):
        x = bf16_bits_to_f32(new["kv_new"][b]).astype(np.float64)
        s = np.abs(x).max() / 448.0
        assert e["kv_sigma"] == s
        y = torch.from_numpy(x / s).to(torch.float8_e4m3fn)
        assert np.array_equal(e["kv"], y.view(torch.uint8).numpy())
        back = s * y.to(torch.float64).numpy()
        assert np.all(np.abs(back - x) <= np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -9) + 1e-300)


# --------------------------------------------------------------------------- IndexCache
def _masked_sdpa(q, K, V, scale, mask):
    """torch SDPA in float64 over all tokens with a boolean [n, T] mask."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]              # [1, H, n, d]
    Kt = torch.from_numpy(K)[None, None].expand(1, q.shape[1], -1, -1)
    Vt = torch.from_numpy(V)[None, None].expand(1, q.shape[1], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=torch.from_numpy(mask)[None, None],
                                                         scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_indexcache_followers_attend_over_the_first_layers_selection():
    """R10: a follower layer's output is dense attention over its own latent rows
    restricted (by a token mask built from the first layer's ids, not by a gather) to
    the selected blocks' tokens at or before the query; the followers' caches differ
    from the first layer's."""
    from long_context_sparse_19_amd.configs import DECODE_INDEXCACHE, scaled_down
    from long_context_sparse_19_amd.inputs import make_inputs, follower_layer, bf16_bits_to_f32
    w = scaled_down(DECODE_INDEXCACHE, 512, batch=2, top_k=16)
    anchor = make_inputs(w)
    followers = [follower_layer(anchor, l) for l in range(1, w.layers)]
    ids, outs = O.indexcache_group(anchor, followers, w.scale, w.dv, w.top_k)
    assert len(outs) == w.layers
    for l, x in enumerate([anchor, *followers]):
        assert l == 0 or not np.array_equal(x.latent, anchor.latent)
        q = bf16_bits_to_f32(x.q).astype(np.float64)
        for b in range(w.batch):
            T = int(x.seq_lens[b])
            KV = bf16_bits_to_f32(x.latent[O.token_rows(x, b, np.arange(T))]).astype(np.float64)
            t = np.arange(T)
            sel = np.zeros(T, bool)
            for j in ids[b][ids[b] >= 0]:
                sel[4 * j: 4 * j + 4] = True
            mask = (sel & (t <= int(x.q_pos[b])))[None]
            ref = _masked_sdpa(q[b:b + 1], KV, KV[:, : w.dv].copy(), w.scale, mask)
            np.testing.assert_allclose(outs[l][0][b], ref[0], rtol=1e-10, atol=1e-12)


def test_indexcache_with_every_block_selected_is_each_layers_own_dense_attention():
    """When the first layer keeps every block, each follower's output is its own dense
    causal attention, whatever the first layer's scores were."""
    from long_context_sparse_19_amd.configs import DECODE_INDEXCACHE, scaled_down
    from long_context_sparse_19_amd.inputs import make_inputs, follower_layer, bf16_bits_to_f32
    w = scaled_down(DECODE_INDEXCACHE, 128, batch=2, top_k=64)
    anchor = make_inputs(w)
    f = follower_layer(anchor, 2)
    _, outs = O.indexcache_group(anchor, [f], w.scale, w.dv, w.top_k)
    q = bf16_bits_to_f32(f.q).astype(np.float64)
    for b in range(w.batch):
        T = int(f.seq_lens[b])
        KV = bf16_bits_to_f32(f.latent[O.token_rows(f, b, np.arange(T))]).astype(np.float64)
        ref = _sdpa_causal(q[b:b + 1], KV, KV[:, : w.dv].copy(), w.scale, np.array([T - 1]))
        np.testing.assert_allclose(outs[1][0][b], ref[0], rtol=1e-11, atol=1e-12)
