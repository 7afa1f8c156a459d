"""Pins of the CPU fp64 oracle against things other than itself.

Each test ties the oracle to a library routine, a closed form, an invariance
of the mathematics, finite differences, or the integer-exact gather encoding,
so that a dropped term, a wrong sign, a wrong index or a transposed operand in
the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import kl_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _rand_case(T=24, d=16, V=64, K=7, seed=0, masked=4, dup=False):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((T, d))
    W = rng.standard_normal((V, d)) / math.sqrt(d) * 2.0
    idx = np.stack([rng.permutation(V)[:K] for _ in range(T)]).astype(np.int32)
    if dup:
        idx[1, 1] = idx[1, 0]
    logp = rng.standard_normal((T, K)) * 2.0 + rng.standard_normal((T, 1)) * 3.0
    mask = np.ones(T, dtype=np.uint8)
    if masked:
        mask[rng.choice(T, masked, replace=False)] = 0
    return H, W, idx, logp, mask


def _torch_dense_loss(H, W, idx, logp, mask):
    """Library form: torch log_softmax over V and kl_div against a dense teacher grid."""
    Ht = torch.as_tensor(H, dtype=torch.float64)
    Wt = torch.as_tensor(W, dtype=torch.float64)
    logq = F.log_softmax(Ht @ Wt.T, dim=1)
    p = torch.softmax(torch.as_tensor(logp, dtype=torch.float64), dim=1)
    m = torch.as_tensor(mask != 0)
    P = torch.zeros_like(logq)
    P.scatter_add_(1, torch.as_tensor(idx, dtype=torch.int64), p)
    kl = F.kl_div(logq[m], P[m], reduction="sum")
    return kl / m.sum()


# ---------------------------------------------------------------- library routines
def test_loss_matches_torch_kl_div_dense_grid():
    H, W, idx, logp, mask = _rand_case()
    ref = _torch_dense_loss(H, W, idx, logp, mask).item()
    got = O.forward(H, W, idx, logp, mask)["loss"]
    assert abs(got - ref) <= 1e-12 * max(1.0, abs(ref))


def test_k_equals_v_permutation_matches_kl_div():
    H, W, _, _, mask = _rand_case(T=10, V=16, K=16, masked=0)
    rng = np.random.default_rng(3)
    idx = np.stack([rng.permutation(16) for _ in range(10)]).astype(np.int32)
    logp = rng.standard_normal((10, 16))
    ref = _torch_dense_loss(H, W, idx, logp, mask).item()
    assert abs(O.forward(H, W, idx, logp, mask)["loss"] - ref) <= 1e-12 * abs(ref)


def test_lse_matches_scipy_logsumexp():
    H, W, idx, logp, mask = _rand_case()
    out = O.forward(H, W, idx, logp, mask)
    ref = scipy.special.logsumexp(H @ W.T, axis=1)
    np.testing.assert_allclose(out["lse"], ref, rtol=1e-13, atol=1e-13)


def test_gradients_match_torch_autograd():
    H, W, idx, logp, mask = _rand_case(dup=True)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    logq = F.log_softmax(Ht @ Wt.T, dim=1)
    p = torch.softmax(torch.as_tensor(logp), dim=1)
    m = torch.as_tensor(mask != 0)
    # per-k sparse form (duplicates kept as separate terms), differentiated by autograd
    lq = torch.gather(logq, 1, torch.as_tensor(idx, dtype=torch.int64))
    loss = -(p * lq)[m].sum() / m.sum() * 0.37
    loss.backward()
    bw = O.backward(H, W, idx, logp, mask, grad_loss=0.37)
    np.testing.assert_allclose(bw["dH"], Ht.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(bw["dW"], Wt.grad.numpy(), rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_golden_closed_forms(case):
    H = np.array(case["H"])
    W = np.eye(case["V"])
    out = O.forward(H, W, np.array(case["idx"]), np.array(case["logp"]), np.array(case["mask"], dtype=np.uint8))
    assert abs(out["loss"] - case["loss"]) <= 1e-14


def test_kl_nonnegative_and_decomposition():
    # KL_t = KL(p || q restricted to the ids and renormalised) - log(sum_k q_{i_k})
    H, W, idx, logp, mask = _rand_case(T=40, masked=0, seed=5)
    out = O.forward(H, W, idx, logp, mask)
    assert (out["row_kl"] >= -1e-12).all()
    _, logq = O.full_log_softmax(H @ W.T)
    lq = np.take_along_axis(logq, idx.astype(np.int64), 1)
    s = np.exp(lq).sum(1)
    l = logp - scipy.special.logsumexp(logp, axis=1, keepdims=True)
    qt = np.exp(lq) / s[:, None]
    kl_inner = scipy.special.rel_entr(np.exp(l), qt).sum(1)
    np.testing.assert_allclose(out["row_kl"], kl_inner - np.log(s), rtol=1e-11, atol=1e-12)
    assert (kl_inner >= -1e-13).all() and (-np.log(s) >= 0).all()


def test_kl_zero_when_student_equals_teacher_and_tail_empty():
    V, K, T = 32, 6, 5
    rng = np.random.default_rng(11)
    idx = np.stack([rng.permutation(V)[:K] for _ in range(T)]).astype(np.int32)
    logp = rng.standard_normal((T, K))
    l = logp - scipy.special.logsumexp(logp, axis=1, keepdims=True)
    c = rng.standard_normal((T, 1)) * 5
    z = np.full((T, V), 0.0) + c - 1000.0          # tail: exp underflows to exactly 0
    np.put_along_axis(z, idx.astype(np.int64), l + c, axis=1)
    out = O.forward(z, np.eye(V), idx, logp + 2.5, None)
    assert np.abs(out["row_kl"]).max() <= 1e-13


def test_kl_equals_minus_log_topk_mass_when_renormalised_student_equals_teacher():
    V, K, T = 40, 5, 4
    rng = np.random.default_rng(12)
    idx = np.stack([rng.permutation(V)[:K] for _ in range(T)]).astype(np.int32)
    logp = rng.standard_normal((T, K))
    l = logp - scipy.special.logsumexp(logp, axis=1, keepdims=True)
    z = np.full((T, V), -1.0)                       # tail logit c - 1 with c = 0
    np.put_along_axis(z, idx.astype(np.int64), l, axis=1)
    out = O.forward(z, np.eye(V), idx, logp, None)
    want = math.log1p((V - K) * math.exp(-1.0))     # -log s with s = 1 / (1 + (V-K)/e)
    np.testing.assert_allclose(out["row_kl"], want, rtol=1e-13)


def test_zero_hidden_states_closed_form():
    H, W, idx, logp, mask = _rand_case(T=12, masked=3, seed=9)
    H[:] = 0.0
    V = W.shape[0]
    fw = O.forward(H, W, idx, logp, mask)
    np.testing.assert_allclose(fw["lse"], math.log(V), rtol=0, atol=1e-14)
    p = scipy.special.softmax(logp, axis=1)
    live = mask != 0
    want = np.mean((math.log(V) + (p * np.log(p)).sum(1))[live])
    assert abs(fw["loss"] - want) <= 1e-13
    bw = O.backward(H, W, idx, logp, mask)
    assert np.abs(bw["dW"]).max() == 0.0
    nv = live.sum()
    for t in range(H.shape[0]):
        want_t = np.zeros(W.shape[1])
        if live[t]:
            want_t = (p[t].sum() * W.mean(0) - (p[t][:, None] * W[idx[t]]).sum(0)) / nv
        np.testing.assert_allclose(bw["dH"][t], want_t, rtol=1e-11, atol=1e-14)


# ---------------------------------------------------------------- finite differences
@pytest.mark.parametrize("gamma,dup,neginf", [(1.0, False, False), (0.73, True, False), (1.9, False, True)])
def test_gradients_finite_differences(gamma, dup, neginf):
    H, W, idx, logp, mask = _rand_case(T=6, d=8, V=32, K=5, masked=2, seed=21, dup=dup)
    if neginf:
        logp[0, 3] = -np.inf
    bw = O.backward(H, W, idx, logp, mask, grad_loss=gamma)
    eps = 1e-6

    def L(Hx, Wx):
        return gamma * O.forward(Hx, Wx, idx, logp, mask)["loss"]

    num_dH = np.zeros_like(H)
    for i in range(H.shape[0]):
        for j in range(H.shape[1]):
            Hp, Hm = H.copy(), H.copy()
            Hp[i, j] += eps
            Hm[i, j] -= eps
            num_dH[i, j] = (L(Hp, W) - L(Hm, W)) / (2 * eps)
    num_dW = np.zeros_like(W)
    for i in range(W.shape[0]):
        for j in range(W.shape[1]):
            Wp, Wm = W.copy(), W.copy()
            Wp[i, j] += eps
            Wm[i, j] -= eps
            num_dW[i, j] = (L(H, Wp) - L(H, Wm)) / (2 * eps)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(bw["dH"], num_dH) <= 1e-6
    assert rel(bw["dW"], num_dW) <= 1e-6


# ---------------------------------------------------------------- invariances
def test_chunk_independence():
    H, W, idx, logp, mask = _rand_case(T=70, seed=2)
    ref_f = O.forward(H, W, idx, logp, mask)
    ref_b = O.backward(H, W, idx, logp, mask)
    for c in (1, 7, 64, 70):
        f = O.forward(H, W, idx, logp, mask, chunk=c)
        b = O.backward(H, W, idx, logp, mask, chunk=c)
        assert abs(f["loss"] - ref_f["loss"]) <= 1e-12 * abs(ref_f["loss"])
        np.testing.assert_allclose(f["row_kl"], ref_f["row_kl"], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(b["dH"], ref_b["dH"], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(b["dW"], ref_b["dW"], rtol=1e-12, atol=1e-15)


def test_teacher_shift_and_permutation_invariance():
    H, W, idx, logp, mask = _rand_case(seed=4)
    base = O.forward(H, W, idx, logp, mask)["loss"]
    shifted = logp + np.random.default_rng(1).standard_normal((logp.shape[0], 1)) * 10
    assert abs(O.forward(H, W, idx, shifted, mask)["loss"] - base) <= 1e-12 * base
    perm = np.random.default_rng(2).permutation(idx.shape[1])
    assert abs(O.forward(H, W, idx[:, perm], logp[:, perm], mask)["loss"] - base) <= 1e-12 * base
    # a different teacher (not a per-row shift) must change it
    assert abs(O.forward(H, W, idx, logp * 1.5, mask)["loss"] - base) > 1e-6


def test_vocab_shift_invariance_and_dw_column_sums():
    H, W, idx, logp, mask = _rand_case(seed=6)
    f0 = O.forward(H, W, idx, logp, mask)
    b0 = O.backward(H, W, idx, logp, mask)
    c = np.random.default_rng(8).standard_normal(W.shape[1])
    f1 = O.forward(H, W + c, idx, logp, mask)
    b1 = O.backward(H, W + c, idx, logp, mask)
    assert abs(f1["loss"] - f0["loss"]) <= 1e-12 * f0["loss"]
    np.testing.assert_allclose(b1["dH"], b0["dH"], rtol=1e-10, atol=1e-13)
    # sum over the vocabulary of G is zero per row, hence sum_v dW[v,:] = 0
    assert np.abs(b0["dW"].sum(0)).max() <= 1e-14 * np.abs(b0["dW"]).max() * W.shape[0]


def test_gather_integer_encoding_is_exact():
    # W[v] = base-256 digits of v, H[t] = (65536, 256, 1): z_{t,v} = v exactly.
    V, K, T, d = 5000, 9, 8, 16
    W = np.zeros((V, d))
    v = np.arange(V)
    W[:, 0], W[:, 1], W[:, 2] = v // 65536, (v // 256) % 256, v % 256
    H = np.zeros((T, d))
    H[:, 0], H[:, 1], H[:, 2] = 65536, 256, 1
    rng = np.random.default_rng(0)
    idx = np.stack([rng.permutation(V)[:K] for _ in range(T)]).astype(np.int32)
    out = O.forward(H, W, idx, rng.standard_normal((T, K)), None)
    assert np.array_equal(out["g"], idx.astype(np.float64))


# ---------------------------------------------------------------- mask semantics
def test_mask_equals_dropping_rows_and_ignores_garbage():
    H, W, idx, logp, mask = _rand_case(T=20, masked=6, seed=13)
    live = mask != 0
    logp_bad = logp.copy()
    logp_bad[~live] = np.nan
    idx_bad = idx.copy()
    idx_bad[~live] = -12345
    f = O.forward(H, W, idx_bad, logp_bad, mask)
    b = O.backward(H, W, idx_bad, logp_bad, mask)
    f_sub = O.forward(H[live], W, idx[live], logp[live], None)
    b_sub = O.backward(H[live], W, idx[live], logp[live], None)
    assert abs(f["loss"] - f_sub["loss"]) <= 1e-13 * f_sub["loss"]
    assert np.abs(b["dH"][~live]).max() == 0.0
    np.testing.assert_allclose(b["dH"][live], b_sub["dH"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(b["dW"], b_sub["dW"], rtol=1e-12, atol=1e-15)


def test_all_masked_gives_zero():
    H, W, idx, logp, _ = _rand_case(T=5, masked=0)
    mask = np.zeros(5, dtype=np.uint8)
    assert O.forward(H, W, idx, logp, mask)["loss"] == 0.0
    b = O.backward(H, W, idx, logp, mask)
    assert not b["dH"].any() and not b["dW"].any()


def test_row_subset_mode_matches_restricted_mask():
    H, W, idx, logp, mask = _rand_case(T=30, masked=5, seed=17)
    rows = np.array([0, 3, 4, 11, 29])
    f_sub = O.forward(H, W, idx, logp, mask, rows=rows)
    f_all = O.forward(H, W, idx, logp, mask)
    np.testing.assert_allclose(f_sub["row_kl"], f_all["row_kl"][rows], rtol=1e-13)
    m2 = np.zeros_like(mask)
    m2[rows] = mask[rows]
    b_sub = O.backward(H, W, idx, logp, mask, rows=rows)
    b_m2 = O.backward(H, W, idx, logp, m2)
    np.testing.assert_allclose(b_sub["dW"], b_m2["dW"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(b_sub["dH"], b_m2["dH"], rtol=1e-12, atol=1e-15)
    assert abs(O.forward(H, W, idx, logp, m2)["loss"] - f_sub["loss"]) <= 1e-13 * f_sub["loss"]


def test_neg_inf_teacher_entry_is_zero_probability():
    H, W, idx, logp, mask = _rand_case(T=4, masked=0, seed=19)
    lp = logp.copy()
    lp[:, -1] = -np.inf
    a = O.forward(H, W, idx, lp, mask)["loss"]
    b = O.forward(H, W, idx[:, :-1], logp[:, :-1], mask)["loss"]
    assert np.isfinite(a) and abs(a - b) <= 1e-13 * b


# ---------------------------------------------------------------- temperature and padding (extensions)
def test_temperature_one_is_the_plain_method():
    H, W, idx, logp, mask = _rand_case(seed=31)
    a, b = O.forward(H, W, idx, logp, mask), O.forward(H, W, idx, logp, mask, temperature=1.0)
    assert a["loss"] == b["loss"] and np.array_equal(a["lse"], b["lse"])
    ga, gb = O.backward(H, W, idx, logp, mask), O.backward(H, W, idx, logp, mask, temperature=1.0)
    assert np.array_equal(ga["dW"], gb["dW"])


def test_temperature_scaling_identity():
    """Scaling H, the teacher log-values and tau by c leaves both softened
    distributions unchanged, so the tau^2-scaled loss grows by exactly c^2 (a
    missing teacher softening or a missing tau^2 breaks this)."""
    H, W, idx, logp, mask = _rand_case(seed=32)
    for tau, c in ((2.0, 3.0), (0.5, 0.25)):
        base = O.forward(H, W, idx, logp, mask, temperature=tau)
        scaled = O.forward(c * H, W, idx, c * logp, mask, temperature=c * tau)
        assert abs(scaled["loss"] - c * c * base["loss"]) <= 1e-12 * abs(c * c * base["loss"])
        np.testing.assert_allclose(scaled["lse"], base["lse"], rtol=1e-12)


def test_temperature_matches_torch_dense_softened_kl():
    """tau^2 * KL(softmax(a/tau) || softmax(z/tau)) through torch's log_softmax / kl_div."""
    H, W, idx, logp, mask = _rand_case(seed=33)
    tau = 2.5
    Ht, Wt = torch.as_tensor(H), torch.as_tensor(W)
    logq = F.log_softmax(Ht @ Wt.T / tau, dim=1)
    p = torch.softmax(torch.as_tensor(logp) / tau, dim=1)
    m = torch.as_tensor(mask != 0)
    P = torch.zeros_like(logq).scatter_add_(1, torch.as_tensor(idx, dtype=torch.int64), p)
    ref = (tau * tau * F.kl_div(logq[m], P[m], reduction="sum") / m.sum()).item()
    assert abs(O.forward(H, W, idx, logp, mask, temperature=tau)["loss"] - ref) <= 1e-12 * abs(ref)


@pytest.mark.parametrize("tau", [2.0, 0.6])
def test_temperature_gradients_finite_differences(tau):
    H, W, idx, logp, mask = _rand_case(T=5, d=6, V=24, K=4, masked=1, seed=34)
    bw = O.backward(H, W, idx, logp, mask, grad_loss=1.3, temperature=tau)
    eps = 1e-6

    def L(Hx, Wx):
        return 1.3 * O.forward(Hx, Wx, idx, logp, mask, temperature=tau)["loss"]

    num_dH = np.zeros_like(H)
    for i in range(H.shape[0]):
        for j in range(H.shape[1]):
            Hp, Hm = H.copy(), H.copy()
            Hp[i, j] += eps
            Hm[i, j] -= eps
            num_dH[i, j] = (L(Hp, W) - L(Hm, W)) / (2 * eps)
    num_dW = np.zeros_like(W)
    for i in range(W.shape[0]):
        for j in range(W.shape[1]):
            Wp, Wm = W.copy(), W.copy()
            Wp[i, j] += eps
            Wm[i, j] -= eps
            num_dW[i, j] = (L(H, Wp) - L(H, Wm)) / (2 * eps)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(bw["dH"], num_dH) <= 1e-6
    assert rel(bw["dW"], num_dW) <= 1e-6


def test_padding_entries_equal_zero_probability_entries():
    """An id below 0 is a padding entry: the same as a valid id with log-value
    -inf, whatever log-value the padding carries."""
    H, W, idx, logp, mask = _rand_case(seed=35)
    pad_idx, pad_logp = idx.copy(), logp.copy()
    pad_idx[2, 3:] = -1
    pad_idx[5, 0] = -7
    pad_logp[2, 3:] = 1e3          # garbage under the padding
    ref_logp = logp.copy()
    ref_logp[2, 3:] = -np.inf
    ref_logp[5, 0] = -np.inf
    for tau in (1.0, 1.7):
        a = O.forward(H, W, pad_idx, pad_logp, mask, temperature=tau)
        b = O.forward(H, W, idx, ref_logp, mask, temperature=tau)
        assert abs(a["loss"] - b["loss"]) <= 1e-13 * abs(b["loss"])
        assert np.isnan(a["g"][2, 3:]).all() and np.isnan(a["g"][5, 0])
        ga = O.backward(H, W, pad_idx, pad_logp, mask, temperature=tau)
        gb = O.backward(H, W, idx, ref_logp, mask, temperature=tau)
        np.testing.assert_allclose(ga["dW"], gb["dW"], rtol=1e-12, atol=1e-16)
        np.testing.assert_allclose(ga["dH"], gb["dH"], rtol=1e-12, atol=1e-16)


# ---------------------------------------------------------------- exact upcast of the storage dtypes
def _bf16_from_words(words: np.ndarray) -> torch.Tensor:
    """A torch bfloat16 tensor holding exactly the given 16-bit patterns."""
    return torch.from_numpy(words.astype(np.uint16).view(np.int16).copy()).view(torch.bfloat16)


def _decode_bf16_words(words: np.ndarray) -> np.ndarray:
    """Hand decode: a bf16 word is the upper half of an IEEE binary32 word."""
    return (words.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_words_of(values) -> np.ndarray:
    """The bf16 patterns of float32 values that bf16 holds exactly (upper halves)."""
    w = np.asarray(values, dtype=np.float32).view(np.uint32)
    assert ((w & 0xFFFF) == 0).all(), "value not representable in bf16"
    return (w >> 16).astype(np.uint16)


def _upcast_case(seed=41):
    """bf16 H and W whose entries a half-precision round trip would change:
    magnitudes above 65504 (fp16 overflows to inf), below 6.1e-5 (fp16
    subnormal or zero), and full 8-bit significands (1 + m/128)."""
    rng = np.random.default_rng(seed)
    T, d, V, K = 7, 8, 24, 5
    sig = 1.0 + rng.integers(0, 128, size=(T, d)) / 128.0               # 8-bit significands
    H = sig * np.exp2(rng.integers(-3, 3, size=(T, d))) * rng.choice([-1.0, 1.0], size=(T, d))
    H[:, 0] = np.array([69632.0, -98304.0, 131072.0, 65536.0, -73728.0, 262144.0, 99328.0])  # > 65504
    Wv = (1.0 + rng.integers(0, 128, size=(V, d)) / 128.0) * np.exp2(rng.integers(-4, 0, size=(V, d)))
    Wv *= rng.choice([-1.0, 1.0], size=(V, d))
    Wv[:, 0] = (1.0 + rng.integers(0, 128, size=V) / 128.0) * np.exp2(-rng.integers(18, 24, size=V))  # < 6.1e-5
    Wv[:, 0] *= rng.choice([-1.0, 1.0], size=V)
    Hw = _bf16_words_of(H.astype(np.float32))
    Ww = _bf16_words_of(Wv.astype(np.float32))
    idx = np.stack([rng.permutation(V)[:K] for _ in range(T)]).astype(np.int32)
    logp = rng.standard_normal((T, K))
    mask = np.ones(T, dtype=np.uint8)
    mask[3] = 0
    return Hw, Ww, idx, logp, mask


def test_bf16_words_are_outside_half_precision():
    # the case really exercises what a half-precision round trip would lose
    Hw, Ww, *_ = _upcast_case()
    Hb, Wb = _bf16_from_words(Hw), _bf16_from_words(Ww)
    assert not torch.equal(Hb.float().half().float(), Hb.float())   # overflow above 65504
    assert not torch.equal(Wb.float().half().float(), Wb.float())   # subnormal / flushed below 6.1e-5


def test_to_f64_decodes_bf16_words_exactly():
    Hw, Ww, *_ = _upcast_case()
    for words in (Hw, Ww):
        got = O.to_f64(_bf16_from_words(words))
        want = _decode_bf16_words(words)
        assert got.dtype == np.float64 and np.array_equal(got, want)
        assert np.array_equal(got, _bf16_from_words(words).to(torch.float64).numpy())


def test_forward_and_backward_on_bf16_tensors_equal_the_decoded_values():
    """The oracle's bf16 entry (torch tensors straight from storage) gives
    exactly the results of the hand-decoded fp64 values."""
    Hw, Ww, idx, logp, mask = _upcast_case()
    Hb, Wb = _bf16_from_words(Hw), _bf16_from_words(Ww)
    Hd, Wd = _decode_bf16_words(Hw), _decode_bf16_words(Ww)
    lp32 = torch.from_numpy(logp.astype(np.float32))
    fa = O.forward(Hb, Wb, idx, lp32, mask)
    fb = O.forward(Hd, Wd, idx, logp.astype(np.float32).astype(np.float64), mask)
    assert np.isfinite(fa["loss"]) and fa["loss"] == fb["loss"]
    assert np.array_equal(fa["lse"], fb["lse"]) and np.array_equal(fa["row_kl"], fb["row_kl"])
    ba = O.backward(Hb, Wb, idx, lp32, mask, grad_loss=0.9)
    bb = O.backward(Hd, Wd, idx, logp.astype(np.float32).astype(np.float64), mask, grad_loss=0.9)
    assert np.isfinite(ba["dW"]).all() and np.array_equal(ba["dH"], bb["dH"])
    assert np.array_equal(ba["dW"], bb["dW"])
    # and the decoded values are not what fp16 storage would have given
    Hh = torch.from_numpy(Hd.astype(np.float32)).half().double().numpy()
    assert not np.isfinite(Hh).all()


def test_to_f64_of_fp32_tensors_and_arrays_is_exact():
    x = np.array([1.0 + 2.0 ** -23, 3.0e38, 1.0e-45, -7.25e-39], dtype=np.float32)
    assert np.array_equal(O.to_f64(torch.from_numpy(x)), x.astype(np.float64))
    assert np.array_equal(O.to_f64(x), x.astype(np.float64))
