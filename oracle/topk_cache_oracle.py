"""CPU fp64 oracle of the teacher top-K cache builder.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests and the benchmark's CPU-baseline leg do.  It shares no code with the
HIP path (nor with the loss oracle beside it).

What it computes: the offline cache the pages describe, in which the teacher
is run once and the K most likely tokens of every position are kept together
with their values (Hugging Face blog "Making Knowledge Distillation Cheap
Enough to Run at Scale", section "Two systems changes"; aimodeling.com article,
section "First cut: remove the teacher from the training loop"):

  1. teacher logits over the whole vocabulary  z_{t,v} = sum_j Ht[t,j] Wt[v,j]
  2. log-probabilities                          log P_{t,v} = z_{t,v} - LSE_t(z)
  3. ids: the K vocabulary entries with the largest z_{t,v} (the most likely
     tokens, softmax being monotone), in decreasing order of z; entries with
     equal logits are taken in increasing id order
  4. values: log P_{t,v} at those ids.

Readings of what the pages leave open:
  * the stored value is the full-vocabulary log-probability: the pages call
    the cache "top-100 logits" (blog title) and "top-100 probabilities"
    (aimodeling.com); a log-probability is the logit shifted by the row's LSE,
    and the loss renormalises over the K entries, so either reading gives the
    same loss;
  * K <= V; rows are independent.

All arithmetic is float64; inputs are upcast exactly from their storage dtype.
``rows`` restricts the work to a subset of positions (large workloads).
"""
from __future__ import annotations

import numpy as np

__all__ = ["to_f64", "teacher_logits", "log_probs", "top_k_ids", "build_cache", "selection_margin"]


def to_f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or a CPU torch tensor (bf16 / fp32) to float64."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if x.is_floating_point():
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def teacher_logits(Ht: np.ndarray, Wt: np.ndarray) -> np.ndarray:
    """Step 1: z = Ht Wt^T, float64."""
    return Ht @ Wt.T


def log_probs(z: np.ndarray):
    """Step 2: (LSE_t, log P_{t,v}) over the full vocabulary (max-shifted)."""
    m = z.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))
    return lse[:, 0], z - lse


def top_k_ids(z: np.ndarray, K: int) -> np.ndarray:
    """Step 3: per row, the K ids with the largest z, decreasing z, ties by increasing id.

    np.lexsort sorts by its last key first: primary key -z (ascending = z
    decreasing), secondary key the id (ascending).
    """
    V = z.shape[1]
    ids = np.arange(V)
    out = np.empty((z.shape[0], K), dtype=np.int64)
    for t in range(z.shape[0]):
        order = np.lexsort((ids, -z[t]))
        out[t] = order[:K]
    return out


def build_cache(Ht, Wt, K: int, rows=None) -> dict:
    """Steps 1-4 for the rows in ``rows`` (all rows by default).

    Returns ``ids`` [R, K] int64, ``logp`` [R, K] (log P at the ids), ``lse`` [R]
    and ``z`` [R, V] (the logits of those rows, for validity checks).
    """
    Ht = to_f64(Ht)
    Wt = to_f64(Wt)
    if rows is not None:
        Ht = Ht[np.asarray(rows, dtype=np.int64)]
    z = teacher_logits(Ht, Wt)
    lse, logP = log_probs(z)
    ids = top_k_ids(z, K)
    return {"ids": ids, "logp": np.take_along_axis(logP, ids, axis=1), "lse": lse, "z": z}


def selection_margin(z: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Per row: min of z over the selected ids minus max of z over the other ids.

    A selection of K ids is a valid top-K exactly when this is >= 0 (the K
    largest values, whatever the order among equal values); with logits that
    carry rounding error, >= -eps.  Rows with K = V return +inf.
    """
    out = np.empty(z.shape[0])
    for t in range(z.shape[0]):
        sel = np.zeros(z.shape[1], dtype=bool)
        sel[np.asarray(ids[t], dtype=np.int64)] = True
        rest = z[t][~sel]
        out[t] = z[t][sel].min() - (rest.max() if rest.size else -np.inf)
    return out
