"""The seeded input recipe, checked property by property (CPU).

The parity tests cannot catch a wrong recipe, since the oracle and the HIP
path read the same bytes; these tests show that the five workloads are the
ones the configurations describe: shapes and dtypes, K distinct uniform ids
per row paired with sorted N(0, 2^2) values log-softmaxed over K, exactly
round(0.05 T) masked rows at random, the document-end zeros of the packed
8K sequence, and a noisy-student teacher that is the top-K of the student
logits plus N(0, 1) noise.
"""
import numpy as np
import pytest
import torch

from chunked_sparse_kl_amd import synth

# (T, d, V, K, dtype, mask, teacher, chunk) of the five configurations
CONFIGS = {
    1: (256, 256, 4096, 16, "f32", "ones", "uniform", 64),
    2: (4096, 3072, 128256, 100, "bf16", "random5", "uniform", 0),
    3: (8192, 3072, 128256, 100, "bf16", "docs4", "noisy_student", 0),
    4: (32768, 2880, 201088, 100, "bf16", "random5", "uniform", 0),
    5: (262144, 3072, 128256, 100, "bf16", "ones", "uniform", 0),
}


@pytest.mark.parametrize("cfg", sorted(CONFIGS))
def test_workload_table(cfg):
    w = synth.WORKLOADS[cfg]
    assert (w.T, w.d, w.V, w.K, w.dtype, w.mask, w.teacher, w.chunk) == CONFIGS[cfg]
    assert w.seed == 1000 + cfg


@pytest.mark.parametrize("cfg", [1, 2, 4, 5])
def test_uniform_teacher_recipe(cfg):
    w = synth.WORKLOADS[cfg]
    ids, logp = synth._uniform_teacher(w.seed, w.T, w.V, w.K)
    assert ids.dtype == torch.int32 and logp.dtype == torch.float32
    assert tuple(ids.shape) == (w.T, w.K) == tuple(logp.shape)
    ids, logp = ids.numpy(), logp.numpy().astype(np.float64)
    # every row: K distinct ids in [0, V)
    assert ids.min() >= 0 and ids.max() < w.V
    s = np.sort(ids, axis=1)
    assert (s[:, 1:] != s[:, :-1]).all()
    # values sorted descending, a log-softmax over K (sum of p = 1)
    assert (np.diff(logp, axis=1) <= 0).all()
    np.testing.assert_allclose(np.log(np.exp(logp).sum(1)), 0.0, atol=2e-6)
    # the values behind the log-softmax are N(0, 2^2): a per-row shift of
    # them, so their within-row spread is that of K draws of std 2
    dev = logp - logp.mean(1, keepdims=True)
    std = np.sqrt((dev ** 2).sum(1).mean() / (w.K - 1))
    assert abs(std - 2.0) < 0.06 * 2.0 + 4.0 / np.sqrt(w.T * w.K)
    # ids uniform over the vocabulary: mean and the count per quarter of V
    n = ids.size
    assert abs(ids.mean() - (w.V - 1) / 2) < 5 * w.V / np.sqrt(12 * n)
    quarters = np.bincount(ids.ravel() * 4 // w.V, minlength=4)
    assert (np.abs(quarters - n / 4) < 6 * np.sqrt(n * 3 / 16)).all()
    # ids are paired with values in draw order, not sorted by id
    assert not (np.diff(ids, axis=1) > 0).all()


@pytest.mark.parametrize("cfg,zeros", [(1, 0), (2, 205), (4, 1638), (5, 0)])
def test_random_mask_counts(cfg, zeros):
    w = synth.WORKLOADS[cfg]
    m = synth._mask(w.seed, w.T, w.mask).numpy()
    assert m.dtype == np.uint8 and m.shape == (w.T,)
    assert set(np.unique(m)) <= {0, 1}
    assert int((m == 0).sum()) == zeros == int(round(0.05 * w.T)) * (w.mask == "random5")
    if zeros:
        # spread over the whole sequence, not a block
        pos = np.nonzero(m == 0)[0]
        assert pos.min() < w.T // 8 and pos.max() > w.T - w.T // 8
        assert np.bincount(pos * 4 // w.T, minlength=4).min() > zeros // 8


def test_packed_documents_mask():
    w = synth.WORKLOADS[3]
    m = synth._mask(w.seed, w.T, w.mask).numpy()
    assert np.array_equal(np.nonzero(m == 0)[0], [2047, 4095, 6143, 8191])


def test_noisy_student_teacher_is_topk_of_noisy_logits():
    T, d, V, K, seed = 40, 64, 3000, 12, 5
    inp = synth.make_custom(T, d, V, K, "bf16", "docs4", "noisy_student", seed=seed)
    H, W = inp["H"], inp["W"]
    # the recipe: fp32 product of the stored bf16 values, plus N(0, 1) noise
    # from the noise sub-stream, one row block at a time
    z = (H.float() @ W.float().t()).double().numpy()
    z += np.random.Generator(np.random.PCG64(seed + 500)).standard_normal((T, V))
    order = np.argsort(-z, axis=1, kind="stable")[:, :K]
    assert np.array_equal(inp["idx"].numpy(), order.astype(np.int32))
    lse = np.log(np.exp(z - z.max(1, keepdims=True)).sum(1)) + z.max(1)
    want = np.take_along_axis(z, order, 1) - lse[:, None]
    np.testing.assert_allclose(inp["logp"].numpy(), want, rtol=0, atol=2e-6)
    # full-vocabulary log-probabilities: the top-K mass is below 1
    assert (np.exp(inp["logp"].double().numpy()).sum(1) < 1.0).all()
    # and the teacher overlaps the student: its ids sit high in the student's own ranking
    zs = (H.float() @ W.float().t()).numpy()
    rank = (zs[:, None, :] > np.take_along_axis(zs, order, 1)[:, :, None]).sum(2)
    assert np.median(rank) < V / 20


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_hidden_states_and_weight_draws(dtype):
    inp = synth.make_custom(512, 256, 4096, 8, dtype, "ones", "uniform", seed=3)
    H, W = inp["H"], inp["W"]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    assert H.dtype == tdt and W.dtype == tdt
    h, wv = H.double().numpy(), W.double().numpy()
    assert abs(h.mean()) < 0.01 and abs(h.std() - 1.0) < 0.01
    assert abs(wv.mean()) < 0.01 / 16 and abs(wv.std() - 256 ** -0.5) < 0.01 / 16
    if dtype == "bf16":
        # rounded from fp32 draws to nearest-even bf16: the stored value is the
        # bf16 nearest to the fp32 draw of the same stream
        draw = np.random.Generator(np.random.PCG64(3)).standard_normal((512, 256), dtype=np.float32)
        near = torch.from_numpy(draw).to(torch.bfloat16)
        assert torch.equal(H, near)
