"""Seeded synthetic inputs for the fused chunked sparse-KL loss head.

This module only draws inputs: student hidden states H, the output-projection
weight W, the teacher's cached top-K ids and log-values, and the row mask.  It
holds none of the loss head's own arithmetic (no student log-softmax, no KL,
no gradient).  Both the CPU oracle's tests and the GPU path's tests and bench
take their inputs from here, so the two sides always see identical bytes.

Workloads follow the pages' toy output-head benchmark and the 8K / 32K heads
("Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused
Chunked KL Loss", Hugging Face blog, section "Scaling to long context
lengths"; arXiv abstract): a teacher cache of the top-100 tokens per position
(blog, section "Two systems changes"), vocabularies of 128,256 and 201,088
(the latter is gpt-oss's, blog section "Why distillation recovery is
expensive").  The pages fix no d, V, K or value distribution for the toy
benchmark; the recipes below are the ones this library is measured on.

Recipe (all draws from numpy PCG64):
  * H ~ N(0, 1), W ~ N(0, 1/d), drawn in float32 and rounded to the storage
    dtype (bf16 round-to-nearest-even via torch, or kept as fp32).
  * "uniform" teacher: per row, K distinct ids uniform over [0, V) (duplicates
    are redrawn), K values ~ N(0, 2^2) sorted descending and paired with the
    ids in draw order, then log-softmaxed over K (stored fp32).
  * "noisy_student" teacher: ids = top-K of (student logits + N(0,1) noise),
    ordered by descending noisy logit; log-values = that noisy row's
    log-softmax over the full vocabulary at those ids (stored fp32).  The
    student logits here are the product of the stored bf16 H and W in fp32.
  * masks: "ones"; "random5" = exactly round(0.05*T) zeros drawn without
    replacement; "docs4" = T split into 4 equal documents, zero at the last
    position of each document (the token whose target crosses a document
    boundary in a packed sequence).
Sub-stream seeds: H +0, W +100, ids +200, values +300, mask +400, noise +500.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_custom"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    V: int
    K: int
    dtype: str          # "bf16" or "f32"
    mask: str           # "ones" | "random5" | "docs4"
    teacher: str        # "uniform" | "noisy_student"
    chunk: int          # 0 = planner chooses
    seed: int


WORKLOADS = {
    1: Workload("tiny-fp32 T=256 d=256 V=4096 K=16", 256, 256, 4096, 16, "f32", "ones", "uniform", 64, 1001),
    2: Workload("toy-head-4k T=4096 d=3072 V=128256 K=100", 4096, 3072, 128256, 100, "bf16", "random5", "uniform", 0, 1002),
    3: Workload("packed-8k T=8192 d=3072 V=128256 K=100", 8192, 3072, 128256, 100, "bf16", "docs4", "noisy_student", 0, 1003),
    4: Workload("head-32k T=32768 d=2880 V=201088 K=100", 32768, 2880, 201088, 100, "bf16", "random5", "uniform", 0, 1004),
    5: Workload("long-256k T=262144 d=3072 V=128256 K=100", 262144, 3072, 128256, 100, "bf16", "ones", "uniform", 0, 1005),
}

_BLOCK = 1 << 24  # elements per draw block (bounds host memory)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal_tensor(rng, rows: int, cols: int, std: float, dtype: str) -> torch.Tensor:
    """rows x cols normal draws, rounded to the storage dtype, drawn in row blocks."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty((rows, cols), dtype=tdt)
    step = max(1, _BLOCK // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        blk = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        out[r0:r1] = torch.from_numpy(blk).to(tdt)
    return out


def _distinct_ids(rng, T: int, V: int, K: int) -> np.ndarray:
    """K distinct ids per row, uniform over [0, V); duplicates are redrawn."""
    ids = rng.integers(0, V, size=(T, K), dtype=np.int64)
    if K > V:
        raise ValueError("K > V")
    if 4 * K > V:  # dense regime: permutation prefix per row
        out = np.empty((T, K), dtype=np.int64)
        for t in range(T):
            out[t] = rng.permutation(V)[:K]
        return out.astype(np.int32)
    while True:
        s = np.sort(ids, axis=1)
        dup_rows = np.nonzero((s[:, 1:] == s[:, :-1]).any(axis=1))[0]
        if dup_rows.size == 0:
            break
        for t in dup_rows:
            row = ids[t]
            _, first = np.unique(row, return_index=True)
            bad = np.setdiff1d(np.arange(K), first)
            row[bad] = rng.integers(0, V, size=bad.size)
    return ids.astype(np.int32)


def _uniform_teacher(seed: int, T: int, V: int, K: int):
    ids = _distinct_ids(_rng(seed + 200), T, V, K)
    vals = _rng(seed + 300).standard_normal((T, K)) * 2.0
    vals = -np.sort(-vals, axis=1)  # descending
    logp = torch.log_softmax(torch.from_numpy(vals), dim=1).to(torch.float32)
    return torch.from_numpy(ids), logp


def _noisy_student_teacher(seed: int, H: torch.Tensor, W: torch.Tensor, K: int):
    """Teacher = top-K of (student logits + N(0,1)); log-values over the full vocabulary."""
    T = H.shape[0]
    V = W.shape[0]
    rng = _rng(seed + 500)
    Hf = H.float()
    Wt = W.float().t().contiguous()
    ids = torch.empty((T, K), dtype=torch.int32)
    logp = torch.empty((T, K), dtype=torch.float32)
    step = 256
    for r0 in range(0, T, step):
        r1 = min(T, r0 + step)
        z = (Hf[r0:r1] @ Wt).double()
        z += torch.from_numpy(rng.standard_normal((r1 - r0, V)))
        lse = torch.logsumexp(z, dim=1, keepdim=True)
        top = torch.topk(z, K, dim=1, largest=True, sorted=True)
        ids[r0:r1] = top.indices.to(torch.int32)
        logp[r0:r1] = (top.values - lse).to(torch.float32)
    return ids, logp


def _mask(seed: int, T: int, kind: str) -> torch.Tensor:
    m = np.ones(T, dtype=np.uint8)
    if kind == "random5":
        nz = int(round(0.05 * T))
        pos = _rng(seed + 400).choice(T, size=nz, replace=False)
        m[pos] = 0
    elif kind == "docs4":
        L = T // 4
        for doc in range(4):
            m[min(T, (doc + 1) * L) - 1] = 0
    elif kind != "ones":
        raise ValueError(kind)
    return torch.from_numpy(m)


def make_custom(T: int, d: int, V: int, K: int, dtype: str = "bf16", mask: str = "ones",
                teacher: str = "uniform", seed: int = 7) -> dict:
    """Inputs for arbitrary sizes with the same recipe (CPU torch tensors)."""
    H = _normal_tensor(_rng(seed + 0), T, d, 1.0, dtype)
    W = _normal_tensor(_rng(seed + 100), V, d, float(d) ** -0.5, dtype)
    if teacher == "uniform":
        idx, logp = _uniform_teacher(seed, T, V, K)
    elif teacher == "noisy_student":
        idx, logp = _noisy_student_teacher(seed, H, W, K)
    else:
        raise ValueError(teacher)
    return {"H": H, "W": W, "idx": idx.contiguous(), "logp": logp.contiguous(),
            "mask": _mask(seed, T, mask)}


def make_inputs(cfg: int) -> dict:
    w = WORKLOADS[cfg]
    out = make_custom(w.T, w.d, w.V, w.K, w.dtype, w.mask, w.teacher, w.seed)
    out["workload"] = w
    return out
