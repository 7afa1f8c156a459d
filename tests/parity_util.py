"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import chunked_sparse_kl_amd as kd
from oracle import kl_oracle as O

# Tolerances of the parity bar: loss relative error, relative Frobenius error of
# dH and dW (bf16 inputs: G and dH are rounded to bf16, 2^-9 relative each;
# fp32 inputs: fp32 accumulation over at most ~2^17 terms).
LOSS_RTOL = 1e-3
GRAD_RTOL = {"bf16": 1e-2, "f32": 1e-5}


def to_device(inp: dict) -> dict:
    dev = torch.device("cuda", 0)
    return {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}


def run_gpu(inp: dict, chunk: int = 0, grad: float = 1.0, mask="inp", gathered=True,
            temperature: float = 1.0) -> dict:
    d = to_device(inp)
    m = d["mask"] if isinstance(mask, str) else (None if mask is None else mask.to(d["H"].device))
    fw = kd.kd_fused_chunked_kl_fwd(d["H"], d["W"], d["idx"], d["logp"], m, chunk=chunk,
                                    gathered=gathered, temperature=temperature)
    g = torch.tensor([grad], dtype=torch.float32, device=d["H"].device)
    dH, dW = kd.kd_fused_chunked_kl_bwd(d["H"], d["W"], d["idx"], d["logp"], m, fw["lse"], g,
                                        plan=fw["plan"], temperature=temperature)
    torch.cuda.synchronize()
    out = {"loss": float(fw["loss"].item()), "lse": fw["lse"].cpu().double().numpy(),
           "row_kl": fw["row_kl"].cpu().double().numpy(), "dH": dH.float().cpu().double().numpy(),
           "dW": dW.cpu().double().numpy(), "plan": fw["plan"]}
    if gathered:
        out["g"] = fw["gathered"].cpu().double().numpy()
    return out


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def subset_rows(n: int, chunk: int, m: int = 256, seed: int = 5) -> np.ndarray:
    """Seeded rows spread over all chunks, including both sides of every chunk boundary."""
    edge = set([0, n - 1])
    for c0 in range(chunk, n, chunk):
        edge.update([c0 - 1, c0])
    edge = sorted(edge)[: m // 2]
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.setdiff1d(np.arange(n), edge), size=max(0, min(m, n) - len(edge)), replace=False)
    return np.sort(np.concatenate([np.array(edge, dtype=np.int64), rest.astype(np.int64)]))


def check_full(inp: dict, gpu: dict, dtype: str, grad: float = 1.0, temperature: float = 1.0):
    """Element-wise comparison with the oracle over all rows (small sizes)."""
    mask = inp["mask"].numpy()
    f = O.forward(inp["H"], inp["W"], inp["idx"].numpy(), inp["logp"], mask, temperature=temperature)
    b = O.backward(inp["H"], inp["W"], inp["idx"].numpy(), inp["logp"], mask, grad_loss=grad,
                   temperature=temperature)
    live = mask != 0
    assert abs(gpu["loss"] - f["loss"]) <= LOSS_RTOL * abs(f["loss"]) + 1e-7, (gpu["loss"], f["loss"])
    np.testing.assert_allclose(gpu["lse"], f["lse"], rtol=2e-6, atol=2e-5)
    np.testing.assert_allclose(gpu["row_kl"][live], f["row_kl"][live], rtol=1e-4, atol=1e-4)
    assert (gpu["row_kl"][~live] == 0).all()
    if "g" in gpu:  # defined on unmasked rows, non-padding entries
        defined = live[:, None] & (inp["idx"].numpy() >= 0)
        np.testing.assert_allclose(gpu["g"][defined], f["g"][defined], rtol=1e-5, atol=1e-4)
    assert rel_fro(gpu["dH"], b["dH"]) <= GRAD_RTOL[dtype], rel_fro(gpu["dH"], b["dH"])
    assert rel_fro(gpu["dW"], b["dW"]) <= GRAD_RTOL[dtype], rel_fro(gpu["dW"], b["dW"])
    assert (gpu["dH"][~live] == 0).all()
    return f, b


def check_subset(inp: dict, chunk: int, dtype: str, rows_m: int = 256):
    """Full-size check on a seeded row subset S: (i) the configuration as given,
    per-row quantities on S; (ii) the mask restricted to S, loss, dH and dW."""
    n, d = inp["H"].shape
    code = kd.KD_BF16 if dtype == "bf16" else kd.KD_F32
    chunk = kd.kd_plan_query(code, n, d, inp["W"].shape[0], inp["idx"].shape[1], chunk)["chunk"]
    S = subset_rows(n, chunk, rows_m)
    mask = inp["mask"].numpy()
    gpu = run_gpu(inp, chunk=chunk)
    f = O.forward(inp["H"], inp["W"], inp["idx"].numpy(), inp["logp"], mask, rows=S)
    live = mask[S] != 0
    np.testing.assert_allclose(gpu["lse"][S], f["lse"], rtol=2e-6, atol=2e-5)
    np.testing.assert_allclose(gpu["row_kl"][S][live], f["row_kl"][live], rtol=1e-4, atol=2e-4)
    np.testing.assert_allclose(gpu["g"][S][live], f["g"][live], rtol=1e-5, atol=2e-4)
    assert np.isfinite(gpu["loss"]) and gpu["loss"] > 0
    res = {"plan": gpu["plan"], "loss_full": gpu["loss"]}
    del gpu
    m2 = np.zeros_like(mask)
    m2[S] = mask[S]
    gpu2 = run_gpu(inp, chunk=chunk, mask=torch.from_numpy(m2), gathered=False)
    b = O.backward(inp["H"], inp["W"], inp["idx"].numpy(), inp["logp"], mask, rows=S)
    res["loss_rel"] = abs(gpu2["loss"] - f["loss"]) / abs(f["loss"])
    res["dH_rel"] = rel_fro(gpu2["dH"], b["dH"])
    res["dW_rel"] = rel_fro(gpu2["dW"], b["dW"])
    assert res["loss_rel"] <= LOSS_RTOL, res
    assert res["dH_rel"] <= GRAD_RTOL[dtype], res
    assert res["dW_rel"] <= GRAD_RTOL[dtype], res
    return res
