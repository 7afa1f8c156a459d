"""Pins of the teacher top-K cache oracle against facts that do not come from it:
pure-Python brute force, closed forms, library routines and invariants."""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import topk_cache_oracle as T


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    Ht = rng.integers(-3, 4, size=(3, 4)).astype(np.float64)
    Wt = rng.integers(-3, 4, size=(9, 4)).astype(np.float64)
    K = 4
    got = T.build_cache(Ht, Wt, K)
    for t in range(3):
        z = [sum(Ht[t, j] * Wt[v, j] for j in range(4)) for v in range(9)]
        m = max(z)
        lse = m + math.log(math.fsum(math.exp(x - m) for x in z))
        order = sorted(range(9), key=lambda v: (-z[v], v))[:K]
        assert list(got["ids"][t]) == order
        np.testing.assert_allclose(got["logp"][t], [z[v] - lse for v in order], rtol=0, atol=1e-12)
        assert abs(got["lse"][t] - lse) < 1e-12


@pytest.mark.parametrize("c", [0.37, -0.21])
def test_linear_logits_closed_form(c):
    # Ht[t] = [1, b_t], Wt[v] = [c v, 1]  ->  z_{t,v} = c v + b_t
    V, K = 50, 7
    b = np.array([0.0, 2.5, -1.0])
    Ht = np.stack([np.ones(3), b], axis=1)
    Wt = np.stack([c * np.arange(V), np.ones(V)], axis=1)
    got = T.build_cache(Ht, Wt, K)
    ids = np.arange(V - 1, V - 1 - K, -1) if c > 0 else np.arange(K)
    log_norm = math.log(math.expm1(c * V) / math.expm1(c))  # log sum_{v<V} e^{c v}
    for t in range(3):
        assert np.array_equal(got["ids"][t], ids)
        np.testing.assert_allclose(got["logp"][t], c * ids - log_norm, rtol=0, atol=1e-12)
        assert abs(got["lse"][t] - (b[t] + log_norm)) < 1e-12


def test_ties_taken_by_increasing_id():
    # Wt[v] = e_{v mod 3}, Ht = [3, 2, 1]: z_v = 3, 2, 1 for v mod 3 = 0, 1, 2
    V, K = 12, 5
    Wt = np.eye(3)[np.arange(V) % 3]
    Ht = np.array([[3.0, 2.0, 1.0]])
    got = T.build_cache(Ht, Wt, K)
    assert list(got["ids"][0]) == [0, 3, 6, 9, 1]
    np.testing.assert_allclose(got["logp"][0], np.array([3, 3, 3, 3, 2]) - got["lse"][0])


def test_invariants_and_library_routines():
    rng = np.random.default_rng(1)
    Ht = rng.standard_normal((6, 16))
    Wt = rng.standard_normal((300, 16))
    K = 20
    got = T.build_cache(Ht, Wt, K)
    z = Ht @ Wt.T
    logP = scipy.special.log_softmax(z, axis=1)
    np.testing.assert_allclose(scipy.special.logsumexp(logP, axis=1), 0.0, atol=1e-12)
    stable = np.argsort(-z, axis=1, kind="stable")[:, :K]   # ties: increasing id
    assert np.array_equal(got["ids"], stable)
    np.testing.assert_allclose(got["logp"], np.take_along_axis(logP, stable, axis=1), rtol=0, atol=1e-12)
    assert (got["logp"] <= 0).all()
    assert (np.diff(got["logp"], axis=1) <= 0).all()
    assert (T.selection_margin(z, got["ids"]) >= 0).all()


def test_selection_margin_detects_an_invalid_set():
    z = np.array([[5.0, 1.0, 4.0, 3.0, 2.0]])
    assert T.selection_margin(z, np.array([[0, 2]]))[0] == 1.0
    assert T.selection_margin(z, np.array([[0, 3]]))[0] == -1.0   # 4.0 left out
    assert T.selection_margin(z, np.array([[0, 1, 2, 3, 4]]))[0] == np.inf


def test_rows_subset_and_bf16_upcast():
    g = torch.Generator().manual_seed(2)
    Ht = torch.randn(10, 32, generator=g).to(torch.bfloat16)
    Wt = torch.randn(200, 32, generator=g).to(torch.bfloat16)
    full = T.build_cache(Ht, Wt, 8)
    rows = [1, 4, 9]
    sub = T.build_cache(Ht, Wt, 8, rows=rows)
    assert np.array_equal(sub["ids"], full["ids"][rows])
    np.testing.assert_array_equal(sub["logp"], full["logp"][rows])
    ref = Ht.double().numpy() @ Wt.double().numpy().T   # bf16 -> fp64 exact
    np.testing.assert_array_equal(full["z"], ref)


def _bf16_words_case(rows: int, cols: int, seed: int) -> np.ndarray:
    """bf16 bit patterns (uint16) of values a half-precision round trip
    would change: magnitudes above 65504 (fp16 overflows) and below 2^-14
    (fp16 subnormals, fewer mantissa bits), with full 7-bit mantissas."""
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, size=(rows, cols)).astype(np.uint16) << 15
    big = rng.integers(127 + 16, 127 + 21, size=(rows, cols))       # 2^16 .. 2^20
    small = rng.integers(127 - 22, 127 - 17, size=(rows, cols))     # 2^-22 .. 2^-18
    expo = np.where(rng.random((rows, cols)) < 0.5, big, small).astype(np.uint16) << 7
    mant = rng.integers(0, 128, size=(rows, cols)).astype(np.uint16)
    return sign | expo | mant


def _decode(words: np.ndarray) -> np.ndarray:
    """Hand decode of bf16 words: the upper half of an fp32 word."""
    return (words.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_bf16_upcast_outside_half_precision():
    Hw, Ww = _bf16_words_case(6, 16, 11), _bf16_words_case(40, 16, 12)
    Ht = torch.from_numpy(Hw.view(np.int16)).view(torch.bfloat16)
    Wt = torch.from_numpy(Ww.view(np.int16)).view(torch.bfloat16)
    assert not torch.equal(Ht.float().half().float(), Ht.float())   # the case exercises fp16's limits
    assert np.array_equal(T.to_f64(Ht), _decode(Hw))
    got = T.build_cache(Ht, Wt, 5)
    ref = T.build_cache(_decode(Hw), _decode(Ww), 5)
    assert np.isfinite(got["z"]).all()
    np.testing.assert_array_equal(got["z"], _decode(Hw) @ _decode(Ww).T)
    assert np.array_equal(got["ids"], ref["ids"]) and np.array_equal(got["logp"], ref["logp"])
