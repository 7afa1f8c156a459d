"""The benchmark's own timed step, checked against the oracle at full size.

bench.py times make_step: the forward and backward calls on one shared
workspace, dW overwritten (never read).  Here that step runs on the 32K-token
workload (T=32768, d=2880, V=201088, K=100, bf16) with the planner's chunk,
exactly as timed, except that the mask keeps only a seeded subset S of rows
(spread over every chunk, both sides of each chunk boundary), so that the
oracle can compute the same loss, dH and dW row by row.  dW starts NaN-filled
and the step runs twice, as after a warm-up.
"""
import numpy as np
import pytest
import torch

import bench
import chunked_sparse_kl_amd as kd
from chunked_sparse_kl_amd import synth
from oracle import kl_oracle as O
from tests.parity_util import GRAD_RTOL, LOSS_RTOL, rel_fro, subset_rows

pytestmark = pytest.mark.gpu


def test_bench_step_matches_oracle_on_subset():
    print("[case] bench step, 32K workload, subset mask", flush=True)
    w = synth.WORKLOADS[bench.WORKLOAD]
    inp = synth.make_inputs(bench.WORKLOAD)
    dev = torch.device("cuda", 0)
    plan = kd.kd_plan_query(kd.KD_BF16, w.T, w.d, w.V, w.K, w.chunk)
    S = subset_rows(w.T, plan["chunk"], 256)
    mask = inp["mask"].numpy()
    m2 = np.zeros_like(mask)
    m2[S] = mask[S]
    H, W = inp["H"].to(dev), inp["W"].to(dev)
    idx, logp = inp["idx"].to(dev), inp["logp"].to(dev)
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=dev)
    dW = torch.full((w.V, w.d), float("nan"), dtype=torch.float32, device=dev)
    grad = torch.ones(1, dtype=torch.float32, device=dev)
    step = bench.make_step(kd, H, W, idx, logp, torch.from_numpy(m2).to(dev), plan, ws, dW, grad)
    step()
    loss, dH = step()
    torch.cuda.synchronize()
    loss = float(loss.item())
    dH = dH.float().cpu().double().numpy()
    dWh = dW.cpu().double().numpy()
    del ws, H, W
    f = O.forward(inp["H"], inp["W"], inp["idx"].numpy(), inp["logp"], mask, rows=S)
    b = O.backward(inp["H"], inp["W"], inp["idx"].numpy(), inp["logp"], mask, rows=S)
    assert abs(loss - f["loss"]) <= LOSS_RTOL * abs(f["loss"]), (loss, f["loss"])
    e_dh, e_dw = rel_fro(dH, b["dH"]), rel_fro(dWh, b["dW"])
    print(f"  loss {loss:.6f} oracle {f['loss']:.6f}  dH rel {e_dh:.2e}  dW rel {e_dw:.2e}", flush=True)
    assert e_dh <= GRAD_RTOL["bf16"] and e_dw <= GRAD_RTOL["bf16"]
    outside = np.ones(w.T, dtype=bool)
    outside[S] = False
    assert not dH[outside].any()
