"""GPU parity of the two comparison variants (dense KL and forward-chunked KL)
against the CPU fp64 oracle and against the fused path.

Both compute the same loss as the fused calls (the pages call the three
mathematically equivalent), from n x V grids the fused path never builds:
dense KL from the full log-probability and teacher-probability grids,
forward-chunked KL from the kept logits.
"""
import numpy as np
import pytest
import torch

import chunked_sparse_kl_amd as kd
from chunked_sparse_kl_amd import synth
from oracle import kl_oracle as O
from tests.parity_util import check_full, rel_fro, run_gpu, to_device

pytestmark = pytest.mark.gpu

VARIANTS = {"dense": (kd.kd_dense_kl_fwd, kd.kd_dense_kl_bwd),
            "forward_chunked": (kd.kd_forward_chunked_kl_fwd, kd.kd_forward_chunked_kl_bwd)}


@pytest.fixture(autouse=True)
def _name(request):
    print(f"[case] {request.node.name}", flush=True)
    yield


def run_variant(name, inp, chunk=0, grad=1.0, mask="inp"):
    fwd, bwd = VARIANTS[name]
    d = to_device(inp)
    m = d["mask"] if isinstance(mask, str) else (None if mask is None else mask.to(d["H"].device))
    fw = fwd(d["H"], d["W"], d["idx"], d["logp"], m, chunk=chunk)
    g = torch.tensor([grad], dtype=torch.float32, device=d["H"].device)
    dH, dW = bwd(d["H"], d["W"], d["idx"], d["logp"], m, fw["lse"], fw["grid"], g, plan=fw["plan"])
    torch.cuda.synchronize()
    out = {"loss": float(fw["loss"].item()), "lse": fw["lse"].cpu().double().numpy(),
           "row_kl": fw["row_kl"].cpu().double().numpy(), "dH": dH.float().cpu().double().numpy(),
           "dW": dW.cpu().double().numpy(), "plan": fw["plan"]}
    del fw
    torch.cuda.empty_cache()
    return out


@pytest.mark.parametrize("name", sorted(VARIANTS))
@pytest.mark.parametrize("chunk", [256, 192, 0])
def test_variant_matches_oracle_small_ragged(name, chunk):
    # several 256-row / 256-vocabulary tiles, a ragged vocabulary tile (V = 1000),
    # a ragged K block (d = 200), a ragged last chunk, 5% masked rows
    inp = synth.make_custom(700, 200, 1000, 20, "bf16", "random5", "uniform", seed=41)
    check_full(inp, run_variant(name, inp, chunk=chunk, grad=0.7), "bf16", grad=0.7)


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_variant_odd_vocabulary(name):
    # V = 1001: the logit rows end inside a 16-byte vector (element-wise stores
    # at the end of each row) and inside the last 256-wide vocabulary tile
    inp = synth.make_custom(333, 136, 1001, 9, "bf16", "random5", "uniform", seed=46)
    check_full(inp, run_variant(name, inp, chunk=128, grad=1.1), "bf16", grad=1.1)


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_variant_below_one_tile(name):
    inp = synth.make_custom(70, 40, 100, 7, "bf16", "random5", "uniform", seed=42)
    check_full(inp, run_variant(name, inp), "bf16")


def test_dense_grid_sums_repeated_ids():
    """A repeated id is one cell of the dense teacher grid, holding the sum of
    its occurrences' p: the dense KL's entropy term is sum_v P log P, the
    oracle's (per cached entry) sum_k p log p.  Everything else, and the
    gradients, agree; the forward-chunked variant keeps the per-entry form."""
    inp = synth.make_custom(300, 128, 900, 12, "bf16", "random5", "uniform", seed=43)
    idx = inp["idx"].numpy()
    idx[3, 1] = idx[3, 0]
    idx[7, 2:5] = idx[7, 1]
    idx[11, [0, 11]] = idx[11, 5]
    inp["idx"] = torch.from_numpy(idx)
    mask = inp["mask"].numpy()
    f = O.forward(inp["H"], inp["W"], idx, inp["logp"], mask)
    l, p = O.renormalise_teacher(inp["logp"].double().numpy())
    P = np.zeros((300, 900))
    np.add.at(P, (np.repeat(np.arange(300), 12), idx.astype(np.int64).ravel()), p.ravel())
    with np.errstate(divide="ignore", invalid="ignore"):
        ent_dense = np.where(P > 0, P * np.log(P), 0.0).sum(1)
    ent_entry = np.where(p > 0, p * l, 0.0).sum(1)
    live = mask != 0
    want = np.where(live, f["row_kl"] + ent_dense - ent_entry, 0.0)
    assert np.abs(want - f["row_kl"])[[3, 7, 11]].min() > 1e-3 or not live[[3, 7, 11]].all()
    dense = run_variant("dense", inp, chunk=128)
    np.testing.assert_allclose(dense["row_kl"], want, rtol=1e-4, atol=1e-4)
    fc = run_variant("forward_chunked", inp, chunk=128)
    np.testing.assert_allclose(fc["row_kl"][live], f["row_kl"][live], rtol=1e-4, atol=1e-4)
    b = O.backward(inp["H"], inp["W"], idx, inp["logp"], mask)
    for out in (dense, fc):
        assert rel_fro(out["dH"], b["dH"]) <= 1e-2 and rel_fro(out["dW"], b["dW"]) <= 1e-2


def test_all_masked_and_masked_rows():
    inp = synth.make_custom(200, 64, 500, 8, "bf16", "ones", "uniform", seed=44)
    inp["mask"][:] = 0
    for name in VARIANTS:
        out = run_variant(name, inp, chunk=64)
        assert out["loss"] == 0.0 and not out["dH"].any() and not out["dW"].any()
        assert (out["row_kl"] == 0).all()


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_variant_agrees_with_fused_at_the_4k_workload(name):
    """The 4K-token toy head (T=4096, d=3072, V=128256, K=100, 5% masked):
    the variant's loss, per-row KL and LSE against the fused path's, and dH,
    dW against the fused path's (both round G to bf16 once)."""
    inp = synth.make_inputs(2)
    fused = run_gpu(inp, chunk=0, gathered=False)
    got = run_variant(name, inp, chunk=0)
    assert got["plan"]["chunk"] == fused["plan"]["chunk"] == 2048
    assert abs(got["loss"] - fused["loss"]) <= 1e-5 * abs(fused["loss"])
    np.testing.assert_allclose(got["lse"], fused["lse"], rtol=1e-6, atol=1e-5)
    live = inp["mask"].numpy() != 0
    np.testing.assert_allclose(got["row_kl"][live], fused["row_kl"][live], rtol=1e-4, atol=2e-4)
    assert rel_fro(got["dH"], fused["dH"]) <= 5e-3 and rel_fro(got["dW"], fused["dW"]) <= 5e-3


@pytest.mark.parametrize("seed", range(8))
def test_variant_random_configuration(seed):
    """Seeded random sizes, chunks, masks and incoming gradients (bf16, the
    variants' dtype), with padding entries; the oracle as the reference."""
    rng = np.random.default_rng(7000 + seed)
    n = int(rng.integers(1, 600))
    d = int(rng.choice([8, 40, 64, 136, 256]))
    K = int(rng.choice([1, 17, 64, 65, 100, 129]))
    V = int(rng.integers(K + 1, 2500))
    inp = synth.make_custom(n, d, V, K, "bf16", "random5" if n >= 20 else "ones", "uniform", seed=7100 + seed)
    idx = inp["idx"].numpy()
    for t in rng.choice(n, size=min(n, 6), replace=False):
        idx[t, int(rng.integers(1, K + 1)):] = -1
    inp["idx"] = torch.from_numpy(idx)
    chunk = int(rng.choice([0, 64, 192, 256]))
    grad = float(rng.uniform(0.3, 1.5)) * (-1.0 if seed % 3 == 1 else 1.0)
    name = sorted(VARIANTS)[seed % 2]
    print(f"[case] {name} n={n} d={d} V={V} K={K} chunk={chunk} grad={grad:.3f}", flush=True)
    check_full(inp, run_variant(name, inp, chunk=chunk, grad=grad), "bf16", grad=grad)


def test_fp32_inputs_are_refused():
    inp = to_device(synth.make_custom(64, 32, 300, 4, "f32", "ones", "uniform", seed=45))
    for name, (fwd, _) in VARIANTS.items():
        with pytest.raises(kd.KdError) as e:
            fwd(inp["H"], inp["W"], inp["idx"], inp["logp"], inp["mask"])
        assert e.value.status == -1
