"""GPU parity against the CPU fp64 oracle on seeded random configurations:
sizes that are ragged against every tile (rows, vocabulary, hidden and
teacher lengths on both sides of the 64-lane and 128-entry boundaries),
chunk sizes, masks, temperatures, incoming gradients of either sign, ids a
row repeats and padding entries, in both storage dtypes."""
import numpy as np
import pytest
import torch

from chunked_sparse_kl_amd import synth
from tests.parity_util import check_full, run_gpu

pytestmark = pytest.mark.gpu

N_CASES = 24


def make_case(seed: int):
    rng = np.random.default_rng(5000 + seed)
    dtype = "f32" if seed % 4 == 0 else "bf16"
    n = int(rng.integers(1, 700))
    d = int(rng.choice([8, 16, 40, 64, 72, 136, 200, 256, 264]))
    K = int(rng.choice([1, 3, 17, 63, 64, 65, 100, 127, 128, 129, 150]))
    V = int(rng.integers(K + 1, 3000))
    mask = str(rng.choice(["ones", "random5", "docs4"])) if n >= 4 else "ones"
    inp = synth.make_custom(n, d, V, K, dtype, mask, "uniform", seed=6000 + seed)
    idx = inp["idx"].numpy()
    for t in rng.choice(n, size=min(n, 8), replace=False):   # repeated ids
        if K > 1:
            src, dst = rng.choice(K, size=2, replace=False)
            idx[t, dst] = idx[t, src]
    for t in rng.choice(n, size=min(n, 8), replace=False):   # padding at the end of a row
        keep = int(rng.integers(1, K + 1))
        idx[t, keep:] = -1
    inp["idx"] = torch.from_numpy(idx)
    chunk = int(rng.choice([0, 64, 128, 192, 256, 512]))
    tau = float(rng.choice([1.0, 1.0, 0.7, 2.0]))
    grad = float(rng.uniform(0.2, 2.0)) * (-1.0 if seed % 5 == 2 else 1.0)
    return inp, dtype, chunk, tau, grad


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration(seed):
    inp, dtype, chunk, tau, grad = make_case(seed)
    n, d = inp["H"].shape
    print(f"[case] seed {seed}: {dtype} n={n} d={d} V={inp['W'].shape[0]} K={inp['idx'].shape[1]} "
          f"chunk={chunk} tau={tau} grad={grad:.3f}", flush=True)
    gpu = run_gpu(inp, chunk=chunk, grad=grad, temperature=tau)
    check_full(inp, gpu, dtype, grad=grad, temperature=tau)
