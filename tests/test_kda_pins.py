"""Pins of the KDA oracle (oracle/kda.py) to closed forms and the delta rule's
defining properties (no GPU needed)."""
import numpy as np
import pytest

from oracle import kda as K


def _orthonormal(n, d, seed):
    q, _ = np.linalg.qr(np.random.default_rng(seed).standard_normal((d, d)))
    return q[:, :n].T                                     # n orthonormal rows


def test_delta_rule_stores_orthonormal_keys_exactly():
    """alpha = 1, beta = 1: writing (k_i, v_i) for orthonormal keys makes the state
    return v_i for k_i (each write leaves the other keys' read-outs untouched)."""
    d = 16
    keys = _orthonormal(6, d, 0)
    vals = np.random.default_rng(1).standard_normal((6, d))
    S = np.zeros((d, d))
    for k, v in zip(keys, vals):
        S, _ = K.delta_step(S, k, k, v, np.ones(d), 1.0)
    np.testing.assert_allclose(keys @ S, vals, atol=1e-12)
    _, o = K.delta_step(S, keys[2], keys[2], S.T @ keys[2], np.ones(d), 1.0)
    np.testing.assert_allclose(o, vals[2] / np.sqrt(d), atol=1e-12)


def test_delta_rule_overwrites_and_interpolates():
    """Writing v2 at a key that holds v1 replaces it (beta = 1); beta in (0, 1) moves
    the read-out the fraction beta of the way to the new value."""
    d = 8
    k = np.zeros(d); k[3] = 1.0
    v1, v2 = np.arange(d, dtype=float), -np.ones(d)
    S, _ = K.delta_step(np.zeros((d, d)), k, k, v1, np.ones(d), 1.0)
    S2, _ = K.delta_step(S, k, k, v2, np.ones(d), 1.0)
    np.testing.assert_allclose(S2.T @ k, v2, atol=1e-14)
    S3, _ = K.delta_step(S, k, k, v2, np.ones(d), 0.25)
    np.testing.assert_allclose(S3.T @ k, 0.75 * v1 + 0.25 * v2, atol=1e-14)


def test_decay_gates_key_channels():
    """alpha = 0 forgets everything before the write; alpha = e_i keeps row i only;
    beta = 0 with alpha = 1 leaves the state as it is and reads S^T q / sqrt(d)."""
    rng = np.random.default_rng(2)
    d = 8
    S = rng.standard_normal((d, d))
    q, k, v = rng.standard_normal((3, d))
    S0, o0 = K.delta_step(S, q, k, v, np.zeros(d), 0.5)
    np.testing.assert_allclose(S0, 0.5 * np.outer(k, v), atol=1e-14)
    np.testing.assert_allclose(o0, 0.5 * (q @ k) * v / np.sqrt(d), atol=1e-13)
    e = np.zeros(d); e[5] = 1.0
    Se, _ = K.delta_step(S, q, k, v, e, 0.0)
    assert np.all(Se[np.arange(d) != 5] == 0) and np.array_equal(Se[5], S[5])
    S1, o1 = K.delta_step(S, q, k, v, np.ones(d), 0.0)
    assert np.array_equal(S1, S)
    np.testing.assert_allclose(o1 * np.sqrt(d), [sum(S[i, j] * q[i] for i in range(d)) for j in range(d)],
                               atol=1e-12)


def test_short_conv_taps_and_silu():
    x = np.array([0.0, 1.0, -2.0, 30.0])
    assert K.silu(0.0) == 0.0
    np.testing.assert_allclose(K.silu(x), [0.0, 1 / (1 + np.exp(-1.0)), -2 / (1 + np.exp(2.0)), 30.0], rtol=1e-12)
    hist = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])      # t-3, t-2, t-1 for 2 channels
    xt = np.array([7.0, 8.0])
    w = np.zeros((2, 4)); w[:, 3] = 1.0
    y, h = K.short_conv(hist, xt, w)
    np.testing.assert_allclose(y, K.silu(xt))
    np.testing.assert_array_equal(h, [[3.0, 4.0], [5.0, 6.0], [7.0, 8.0]])
    w = np.zeros((2, 4)); w[0, 0] = 1.0; w[1, :] = [1.0, -1.0, 0.5, 2.0]
    y, _ = K.short_conv(hist, xt, w)
    np.testing.assert_allclose(y, K.silu([1.0, 2.0 - 4.0 + 3.0 + 16.0]))


def test_l2norm_unit_rows():
    x = np.random.default_rng(3).standard_normal((5, 128))
    n = np.linalg.norm(K.l2norm(x), axis=1)
    np.testing.assert_allclose(n, np.linalg.norm(x, axis=1) / np.sqrt(np.linalg.norm(x, axis=1) ** 2 + K.EPS))


def test_decode_step_wiring_closed_form():
    """Zero state, alpha = 1, beta = 1, conv weights on the current tap: after one step
    S = k^ v^T and o = (q^ . k^) v^ / sqrt(dk) with q^, k^ the normalised SiLU of x_q,
    x_k and v^ the SiLU of x_v (catches swapped q / k / v paths).  With the weights on
    the previous tap, the second step sees the first step's inputs."""
    rng = np.random.default_rng(4)
    B, H, d = 2, 3, 8
    xq, xk, xv = rng.standard_normal((3, B, H * d))
    w = np.zeros((3, H * d, 4)); w[:, :, 3] = 1.0
    S, cs, o = K.decode_step(np.zeros((B, H, d, d)), np.zeros((B, 3, 3, H * d)), xq, xk, xv,
                             np.ones((B, H, d)), np.ones((B, H)), w)
    for b in range(B):
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            qh, kh, vh = K.l2norm(K.silu(xq[b, sl])), K.l2norm(K.silu(xk[b, sl])), K.silu(xv[b, sl])
            np.testing.assert_allclose(S[b, h], np.outer(kh, vh), atol=1e-14)
            np.testing.assert_allclose(o[b, h], (qh @ kh) * vh / np.sqrt(d), atol=1e-14)
    np.testing.assert_array_equal(cs[:, 0, 2], xq)
    np.testing.assert_array_equal(cs[:, 2, 2], xv)
    w2 = np.zeros((3, H * d, 4)); w2[:, :, 2] = 1.0
    yq, yk, yv = rng.standard_normal((3, B, H * d))
    S2, _, o2 = K.decode_step(np.zeros((B, H, d, d)), cs, yq, yk, yv, np.ones((B, H, d)), np.ones((B, H)), w2)
    np.testing.assert_allclose(S2[1, 2], np.outer(K.l2norm(K.silu(xk[1, 2 * d:])), K.silu(xv[1, 2 * d:])), atol=1e-14)


def test_prefill_chunk_is_the_token_recurrence():
    """prefill_chunk over T tokens is T decode steps in order (state, taps and every
    output), and a chunk of no tokens changes nothing."""
    rng = np.random.default_rng(5)
    B, H, d, T = 2, 2, 8, 5
    S0 = rng.standard_normal((B, H, d, d))
    cs0 = rng.standard_normal((B, 3, 3, H * d))
    xq, xk, xv = (rng.standard_normal((B, T, H * d)) for _ in range(3))
    al = rng.uniform(0.5, 1.0, (B, T, H, d))
    be = rng.uniform(0.0, 1.0, (B, T, H))
    w = rng.standard_normal((3, H * d, 4))
    S, cs, o = K.prefill_chunk(S0, cs0, xq, xk, xv, al, be, w)
    S2, cs2 = S0, cs0
    for t in range(T):
        S2, cs2, ot = K.decode_step(S2, cs2, xq[:, t], xk[:, t], xv[:, t], al[:, t], be[:, t], w)
        np.testing.assert_array_equal(o[:, t], ot)
    np.testing.assert_array_equal(S, S2)
    np.testing.assert_array_equal(cs, cs2)
    S3, cs3, o3 = K.prefill_chunk(S0, cs0, xq[:, :0], xk[:, :0], xv[:, :0], al[:, :0], be[:, :0], w)
    assert o3.shape == (B, 0, H, d)
    np.testing.assert_array_equal(S3, S0)
    np.testing.assert_array_equal(cs3, cs0)
