"""The forward that allocates nothing, against the regular forward.

kd_fused_chunked_kl_fwd_noalloc runs the regular forward's kernels on the
library's per-GPU scratch array instead of a caller workspace, so its loss,
per-row LSE, per-row KL and gathered logits must equal the regular call's bit
for bit (both are also independent of the chunk).  Two calls in a row, the
second on a smaller problem, show that the contents the first leaves in the
shared scratch do not leak into the second.
"""
import ctypes

import numpy as np
import pytest
import torch

import chunked_sparse_kl_amd as kd
from chunked_sparse_kl_amd import synth

pytestmark = pytest.mark.gpu


def _compare(inp, chunk):
    dev = torch.device("cuda", 0)
    H, W = inp["H"].to(dev), inp["W"].to(dev)
    idx, logp, mask = inp["idx"].to(dev), inp["logp"].to(dev), inp["mask"].to(dev)
    n, K = idx.shape
    ref = kd.kd_fused_chunked_kl_fwd(H, W, idx, logp, mask, chunk=chunk, row_kl=True, gathered=True)
    torch.cuda.synchronize()
    outs = {"loss": torch.full((1,), float("nan"), device=dev), "lse": torch.full((n,), float("nan"), device=dev),
            "row_kl": torch.full((n,), float("nan"), device=dev),
            "gathered": torch.full((n, K), float("nan"), device=dev)}
    # nothing is allocated through torch either: its count of allocation
    # requests (which frees by the garbage collector never change) stays put
    requests = torch.cuda.memory_stats(dev)["allocation.all.allocated"]
    got = kd.kd_fused_chunked_kl_fwd_noalloc(H, W, idx, logp, mask, chunk=chunk, **outs)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats(dev)["allocation.all.allocated"] == requests
    assert torch.equal(got["loss"], ref["loss"]) and torch.equal(got["lse"], ref["lse"])
    assert torch.equal(got["row_kl"], ref["row_kl"])
    live = (mask != 0)[:, None] & (idx >= 0)               # gathered values are defined there
    assert torch.equal(got["gathered"][live], ref["gathered"][live])
    assert torch.isfinite(got["loss"]).all() and got["loss"].item() > 0
    return got


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_forward_equals_regular_forward_on_two_calls(dtype):
    print(f"[case] no-alloc forward, {dtype}, two calls", flush=True)
    big = synth.make_custom(2100, 320, 5000, 40, dtype, "random5", "uniform", seed=31)
    small = synth.make_custom(700, 192, 3000, 24, dtype, "ones", "uniform", seed=32)
    _compare(big, chunk=0)
    _compare(small, chunk=256)          # smaller problem on the scratch the first call left behind


def test_noalloc_forward_at_the_32k_shape():
    # the largest loss-head workload whose forward fits the scratch: T=32768, d=2880, V=201088, K=100
    print("[case] no-alloc forward, 32K workload", flush=True)
    p = kd.kd_plan_query(kd.KD_BF16, 32768, 2880, 201088, 100, 8192, 1)
    assert p["fwd_workspace_bytes"] <= kd.KD_NOALLOC_SCRATCH_BYTES
    inp = synth.make_inputs(4)
    got = _compare(inp, chunk=0)
    small = synth.make_custom(300, 2880, 201088, 100, "bf16", "random5", "uniform", seed=33)
    _compare(small, chunk=0)
    del got


def test_noalloc_forward_rejects_problems_beyond_its_scratch():
    lib = kd.lib()
    fake = ctypes.c_void_p(4096)
    # 256K tokens: the per-row teacher buffers alone exceed the scratch
    rc = lib.kd_fused_chunked_kl_fwd_noalloc(0, fake, fake, fake, fake, None, 262144, 3072, 128256, 100, 0,
                                             1.0, fake, fake, None, None, None)
    assert rc == -2 and b"no-allocation" in lib.kd_last_error_message()
    # an explicit chunk whose partials do not fit
    rc = lib.kd_fused_chunked_kl_fwd_noalloc(0, fake, fake, fake, fake, None, 200000, 64, 2000000, 8, 200000,
                                             1.0, fake, fake, None, None, None)
    assert rc == -2 and b"no-allocation" in lib.kd_last_error_message()
