"""Pins of the Gated DeltaNet-2 oracle (oracle/gdn2.py) to results fixed by the
mathematics rather than by the oracle itself:

* with no erase (b = 0) and no decay (g = 0) the recurrence is causal linear
  attention, o_t = scale (q_t^T S0 + sum_{j<=t} (q_t . k_j) w_j * v_j), computed
  here as one masked matrix product;
* with no writes (b = 0, w = 0) the state only decays:
  S_t = diag(exp(sum_{s<=t} g_s)) S0, o_t = scale (q_t * exp(G_t))^T S0;
* the delta rule's write: for a unit key k, erase gate b = beta (all key dims)
  and write gate 1, one token maps S' = diag(exp(g)) S0 to S_1 with
  S_1^T k = v + (1 - beta) S'^T k, whatever S0 and g are (beta = 1 stores v at
  key k exactly), which fails if the erase reads the undecayed state, if the
  decay follows the write, or if b is dropped;
* the chunked (WY) regrouping equals the token-by-token recurrence for chunk
  lengths 1, 3, 16, 64 and longer than the sequence.
"""
import numpy as np
import pytest

from oracle import gdn2


def _inputs(B=2, H=3, T=37, K=8, V=6, seed=0, unit_k=True):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((B, H, T, K)), rng.standard_normal((B, H, T, K))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    g = -0.3 * np.abs(rng.standard_normal((B, H, T, K)))
    b = rng.uniform(0.0, 1.0, (B, H, T, K))
    v, w = rng.standard_normal((B, H, T, V)), rng.uniform(0.5, 1.5, (B, H, T, V))
    S0 = rng.standard_normal((B, H, K, V))
    return q, k, v, g, b, w, S0


def test_no_erase_no_decay_is_causal_linear_attention():
    q, k, v, g, b, w, S0 = _inputs(seed=1)
    o, S = gdn2.recurrent(q, k, v, np.zeros_like(g), np.zeros_like(b), w, S0, scale=0.5)
    T = q.shape[2]
    att = np.einsum("bhtk,bhsk->bhts", q, k) * np.tril(np.ones((T, T)))
    ref = 0.5 * (att @ (w * v) + q @ S0)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S0 + np.swapaxes(k, 2, 3) @ (w * v), rtol=1e-12, atol=1e-12)


def test_no_writes_only_decay():
    q, k, v, g, b, w, S0 = _inputs(seed=2)
    o, S = gdn2.recurrent(q, k, v, g, np.zeros_like(b), np.zeros_like(w), S0, scale=1.3)
    G = np.cumsum(g, axis=2)
    np.testing.assert_allclose(S, np.exp(G[:, :, -1])[..., None] * S0, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o, 1.3 * (q * np.exp(G)) @ S0, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("beta", [1.0, 0.3])
def test_delta_rule_write_at_a_unit_key(beta):
    q, k, v, g, b, w, S0 = _inputs(T=1, seed=3)
    b = np.full_like(b, beta)
    _, S1 = gdn2.recurrent(q, k, v, g, b, np.ones_like(w), S0)
    Sp = np.exp(g[:, :, 0])[..., None] * S0
    lhs = np.einsum("bhkv,bhk->bhv", S1, k[:, :, 0])
    rhs = v[:, :, 0] + (1.0 - beta) * np.einsum("bhkv,bhk->bhv", Sp, k[:, :, 0])
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 3, 16, 64, 50])
def test_chunked_equals_recurrent(chunk):
    q, k, v, g, b, w, S0 = _inputs(seed=4)
    o1, S1 = gdn2.recurrent(q, k, v, g, b, w, S0, scale=0.7)
    o2, S2 = gdn2.chunked(q, k, v, g, b, w, S0, scale=0.7, chunk=chunk)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S2, S1, rtol=1e-10, atol=1e-12)


def test_zero_initial_state_default():
    q, k, v, g, b, w, S0 = _inputs(T=5, seed=5)
    o1, S1 = gdn2.recurrent(q, k, v, g, b, w)
    o2, S2 = gdn2.recurrent(q, k, v, g, b, w, np.zeros_like(S0))
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
