"""CPU fp64 oracle for the fused chunked sparse-KL distillation loss head.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests, the smoke check and the benchmark's CPU-baseline leg do.  It shares
no code with the HIP path.

What it computes (the "dense KL" formulation of the pages, which they state is
mathematically equivalent to the forward-chunked and fused chunked variants:
Hugging Face blog "Making Knowledge Distillation Cheap Enough to Run at
Scale", section "Two systems changes"; Japanese summary on aib.vote, paragraph
comparing Dense KL, Forward-chunked KL and Fused chunked KL):

  For each position t, with teacher ids i_{t,k} and cached log-values a_{t,k}
  (k < K, the offline top-K cache of the blog's "Two systems changes"):
   1. student logits over the whole vocabulary  z_{t,v} = sum_j H[t,j] W[v,j]
   2. full-vocabulary log-softmax               log q_{t,v} = z_{t,v} - LSE_t(z)
   3. teacher renormalised over its K entries   l_{t,k} = a_{t,k} - LSE_k(a_t),
                                                p_{t,k} = exp(l_{t,k})
   4. KL_t = sum_k p_{t,k} (l_{t,k} - log q_{t,i_{t,k}})   (0 * log 0 := 0)
   5. loss = (1/N_valid) sum_{t: mask_t != 0} KL_t   (0 when N_valid = 0)
   6. gradient w.r.t. the logits (the closed form the blog mentions in its
      closing paragraph but does not print; it follows from step 2 and 4):
        G_{t,v} = gamma * [mask_t] / N_valid * (S_t q_{t,v} - sum_k p_{t,k} [i_{t,k} = v])
      with S_t = sum_k p_{t,k} and gamma the upstream gradient of the loss;
      dH = G W  and  dW = G^T H.

Readings of what the pages leave open (each is listed with its reason in the
design notes of the repository):
  * no tail bucket: the student is normalised over all V, the teacher's mass
    lives only on its K ids (renormalised), the KL sums over those K ids;
  * forward KL(teacher || student), mean over unmasked rows;
  * masked rows are skipped entirely (their ids / values may be garbage);
  * duplicate ids in a row are summed in the gradient (scatter-add);
  * a log-value of -inf is a zero-probability entry; an id below 0 marks a
    padding entry (rows with fewer than K cached entries), treated the same
    way whatever its log-value.

Temperature (an extension; the pages never mention one, the default 1 is the
method as described): the usual soft-target distillation with both sides
softened and the loss scaled back by tau^2, i.e. steps 2-5 on z / tau and
a / tau, loss = tau^2 * mean KL, and hence
  G_{t,v} = gamma * tau * [mask_t] / N_valid * (S_t q_{t,v} - sum_k p_{t,k} [i_{t,k} = v])
with q and p the softened distributions.  ``lse`` is then LSE_t(z / tau) and
``row_kl`` is tau^2 KL_t.

All arithmetic is float64; inputs are upcast exactly from their storage dtype.
``rows`` restricts the work to a subset of positions (for the large
workloads, where the full logit matrix would not fit in host memory).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "to_f64", "student_logits", "full_log_softmax", "renormalise_teacher",
    "gather", "kl_rows", "n_valid", "forward", "backward",
]


def to_f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or a CPU torch tensor (bf16 / fp32) to float64."""
    if hasattr(x, "detach"):  # torch tensor: bf16 -> fp32 is exact, fp32 -> fp64 is exact
        x = x.detach().cpu()
        if x.is_floating_point():
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def student_logits(H: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Step 1: z = H W^T over the full vocabulary, float64."""
    return H @ W.T


def full_log_softmax(z: np.ndarray):
    """Step 2: returns (LSE_t, log q_{t,v}) over the full vocabulary (max-shifted)."""
    m = z.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))
    return lse[:, 0], z - lse


def renormalise_teacher(a: np.ndarray):
    """Step 3: (l, p) with l = a - LSE over the K entries, p = exp(l).

    Entries equal to -inf get p = 0 and l = -inf.  A row whose entries are all
    -inf has no distribution and yields NaN.
    """
    A = a.max(axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):
        lam = A + np.log(np.exp(a - A).sum(axis=1, keepdims=True))
        l = a - lam
    p = np.exp(l)
    return l, p


def gather(z_or_logq: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Values of a [rows, V] matrix at each row's teacher ids -> [rows, K]."""
    return np.take_along_axis(z_or_logq, idx.astype(np.int64), axis=1)


def kl_rows(p: np.ndarray, l: np.ndarray, logq_ids: np.ndarray) -> np.ndarray:
    """Step 4: KL_t = sum_k p (l - log q at the teacher id), with 0 * anything := 0."""
    with np.errstate(invalid="ignore"):
        terms = np.where(p > 0, p * (l - logq_ids), 0.0)
    return terms.sum(axis=1)


def n_valid(mask: np.ndarray) -> int:
    return int(np.count_nonzero(np.asarray(mask)))


def _row_blocks(rows: np.ndarray, chunk):
    if chunk is None or chunk <= 0:
        chunk = max(1, rows.size)
    for s in range(0, rows.size, chunk):
        yield rows[s:s + chunk]


def _teacher_inputs(idx: np.ndarray, a: np.ndarray, temperature: float):
    """Padding entries (id < 0) become zero-probability entries at id 0; the
    log-values are softened by the temperature."""
    pad = idx < 0
    a = np.where(pad, -np.inf, a / temperature)
    return np.where(pad, 0, idx), a, pad


def forward(H, W, idx, logp, mask=None, chunk=None, rows=None, temperature: float = 1.0) -> dict:
    """Loss and per-row quantities.

    Returns a dict with: ``loss`` (float; over the rows in ``rows`` that are
    unmasked, divided by their count), ``row_kl`` [R] (0 for masked rows),
    ``lse`` [R], ``g`` [R, K] (student logits at the teacher ids; NaN, i.e.
    undefined, on masked rows, whose ids are never read), ``rows``.
    ``chunk`` processes the rows in independent blocks of that many rows.
    With a temperature, ``lse`` is LSE(z / tau), ``row_kl`` is tau^2 KL_t and
    ``g`` stays the raw logit z; padding entries have g = NaN.
    """
    H = to_f64(H)
    W = to_f64(W)
    idx, a_all, pad = _teacher_inputs(np.asarray(idx), to_f64(logp), float(temperature))
    tau = float(temperature)
    T = H.shape[0]
    mask = np.ones(T, dtype=np.uint8) if mask is None else np.asarray(mask)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    row_kl = np.zeros(rows.size)
    lse = np.zeros(rows.size)
    g = np.zeros((rows.size, idx.shape[1]))
    pos = 0
    for blk in _row_blocks(rows, chunk):
        z = student_logits(H[blk], W)
        lse_b, logq = full_log_softmax(z / tau)
        live = mask[blk] != 0
        kl = np.zeros(blk.size)
        g_b = np.full((blk.size, idx.shape[1]), np.nan)  # undefined for masked rows
        if live.any():
            ids_live = idx[blk][live]
            g_b[live] = np.where(pad[blk][live], np.nan, gather(z[live], ids_live))
            l, p = renormalise_teacher(a_all[blk][live])
            kl[live] = tau * tau * kl_rows(p, l, gather(logq[live], ids_live))
        row_kl[pos:pos + blk.size] = kl
        lse[pos:pos + blk.size] = lse_b
        g[pos:pos + blk.size] = g_b
        pos += blk.size
    nv = n_valid(mask[rows])
    loss = float(row_kl.sum() / nv) if nv > 0 else 0.0
    return {"loss": loss, "row_kl": row_kl, "lse": lse, "g": g, "rows": rows, "n_valid": nv}


def backward(H, W, idx, logp, mask=None, grad_loss: float = 1.0, chunk=None, rows=None,
             temperature: float = 1.0) -> dict:
    """dH [T, d] and dW [V, d] of ``grad_loss * loss`` (step 6).

    With ``rows`` given, only those rows contribute (the others are treated as
    masked), which is exactly the gradient of the loss restricted to them.
    """
    H = to_f64(H)
    W = to_f64(W)
    idx, a_all, _ = _teacher_inputs(np.asarray(idx), to_f64(logp), float(temperature))
    tau = float(temperature)
    T, d = H.shape
    V = W.shape[0]
    mask = np.ones(T, dtype=np.uint8) if mask is None else np.asarray(mask)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    live_rows = rows[mask[rows] != 0]
    nv = live_rows.size
    dH = np.zeros((T, d))
    dW = np.zeros((V, d))
    if nv == 0:
        return {"dH": dH, "dW": dW, "n_valid": 0}
    for blk in _row_blocks(live_rows, chunk):
        z = student_logits(H[blk], W)
        _, logq = full_log_softmax(z / tau)
        q = np.exp(logq)
        _, p = renormalise_teacher(a_all[blk])
        S = p.sum(axis=1)
        G = S[:, None] * q
        scatter = np.zeros_like(G)
        r = np.repeat(np.arange(blk.size), idx.shape[1])
        np.add.at(scatter, (r, idx[blk].astype(np.int64).ravel()), p.ravel())
        G = (grad_loss * tau / nv) * (G - scatter)
        dH[blk] = G @ W
        dW += G.T @ H[blk]
    return {"dH": dH, "dW": dW, "n_valid": nv}
