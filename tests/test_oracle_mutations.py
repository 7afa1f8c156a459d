"""Sensitivity of the oracles' pins: plausible mistakes planted in a copy of
an oracle's source (on the CPU, one at a time) each make at least one of its
pins fail (tests/test_oracle_pins.py for the loss oracle,
tests/test_topk_oracle_pins.py for the cache builder's), while the unchanged
sources pass them all.

A mutant is the oracle module's text with one line edited, executed as a
fresh module and handed to the pins in place of the real one for the
duration of the check.  (Edits that are identities of the mathematics are
not mistakes and are not listed: for instance subtracting the column mean of
W in dH changes nothing, because every row of G sums to zero.)
"""
import json
import os
import types

import pytest

import tests.test_oracle_pins as P
import tests.test_topk_oracle_pins as PT

SRC = os.path.join(os.path.dirname(__file__), "..", "oracle", "kl_oracle.py")
SRC_TOPK = os.path.join(os.path.dirname(__file__), "..", "oracle", "topk_cache_oracle.py")

# (name, text in the oracle, replacement): each edit is a mistake a reader of
# the pages could make while writing the oracle.
MUTATIONS = [
    ("teacher not renormalised over K",
     "lam = A + np.log(np.exp(a - A).sum(axis=1, keepdims=True))", "lam = A"),
    ("KL terms with the wrong sign",
     "terms = np.where(p > 0, p * (l - logq_ids), 0.0)", "terms = np.where(p > 0, p * (logq_ids - l), 0.0)"),
    ("gather one id off",
     "return np.take_along_axis(z_or_logq, idx.astype(np.int64), axis=1)",
     "return np.take_along_axis(z_or_logq, (idx.astype(np.int64) + 1) % z_or_logq.shape[1], axis=1)"),
    ("mean over all rows instead of the unmasked ones",
     "loss = float(row_kl.sum() / nv) if nv > 0 else 0.0",
     "loss = float(row_kl.sum() / row_kl.size) if nv > 0 else 0.0"),
    ("temperature squared factor dropped from the KL",
     "kl[live] = tau * tau * kl_rows(", "kl[live] = tau * kl_rows("),
    ("temperature applied the wrong way to the teacher",
     "a = np.where(pad, -np.inf, a / temperature)", "a = np.where(pad, -np.inf, a * temperature)"),
    ("temperature factor dropped from G",
     "G = (grad_loss * tau / nv) * (G - scatter)", "G = (grad_loss / nv) * (G - scatter)"),
    ("teacher scatter added instead of subtracted",
     "G = (grad_loss * tau / nv) * (G - scatter)", "G = (grad_loss * tau / nv) * (G + scatter)"),
    ("dW with the wrong sign",
     "dW += G.T @ H[blk]", "dW -= G.T @ H[blk]"),
    ("dH written to the wrong rows",
     "dH[blk] = G @ W", "dH[:blk.size] = G @ W"),
    ("dW from the wrong rows of H",
     "dW += G.T @ H[blk]", "dW += G.T @ H[:blk.size]"),
    ("student normalised without its row maximum shift being undone",
     "lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))",
     "lse = np.log(np.exp(z - m).sum(axis=1, keepdims=True))"),
    ("bf16 upcast through half precision",
     "x = x.float()", "x = x.half().float()"),
    ("zero-probability entries not set aside (0 * -inf)",
     "terms = np.where(p > 0, p * (l - logq_ids), 0.0)", "terms = p * (l - logq_ids)"),
    ("student not softened by the temperature in the forward",
     "lse_b, logq = full_log_softmax(z / tau)", "lse_b, logq = full_log_softmax(z)"),
    ("student not softened by the temperature in the backward",
     "_, logq = full_log_softmax(z / tau)", "_, logq = full_log_softmax(z)"),
    ("log-probability stored as the gathered logit",
     "g_b[live] = np.where(pad[blk][live], np.nan, gather(z[live], ids_live))",
     "g_b[live] = np.where(pad[blk][live], np.nan, gather(logq[live], ids_live))"),
    ("teacher entries scattered into the wrong rows",
     "r = np.repeat(np.arange(blk.size), idx.shape[1])", "r = np.tile(np.arange(blk.size), idx.shape[1])"),
    ("masked rows kept in the gradient",
     "live_rows = rows[mask[rows] != 0]", "live_rows = rows"),
    ("gradient divided by all rows",
     "nv = live_rows.size", "nv = rows.size"),
]


# the same for the cache builder's oracle
MUTATIONS_TOPK = [
    ("ties taken by decreasing id",
     "order = np.lexsort((ids, -z[t]))", "order = np.lexsort((-ids, -z[t]))"),
    ("smallest logits kept instead of the largest",
     "order = np.lexsort((ids, -z[t]))", "order = np.lexsort((ids, z[t]))"),
    ("stored value is the logit, not the log-probability",
     'return {"ids": ids, "logp": np.take_along_axis(logP, ids, axis=1), "lse": lse, "z": z}',
     'return {"ids": ids, "logp": np.take_along_axis(z, ids, axis=1), "lse": lse, "z": z}'),
    ("log-probabilities without the row maximum",
     "lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))",
     "lse = np.log(np.exp(z - m).sum(axis=1, keepdims=True))"),
    ("rows subset ignored",
     "Ht = Ht[np.asarray(rows, dtype=np.int64)]", "Ht = Ht"),
    ("selection margin against the selected ids",
     "rest = z[t][~sel]", "rest = z[t][sel]"),
    ("bf16 upcast through half precision",
     "x = x.float()", "x = x.half().float()"),
]


def _topk_pin_calls():
    calls = []
    for name, fn in vars(PT).items():
        if not (name.startswith("test_") and callable(fn)):
            continue
        if name == "test_linear_logits_closed_form":
            calls += [(f"{name}[{c}]", lambda c=c: PT.test_linear_logits_closed_form(c)) for c in (0.37, -0.21)]
        else:
            calls.append((name, fn))
    return calls


def _pin_calls():
    cases = json.load(open(P.GOLDEN))["cases"]
    calls = []
    for name, fn in vars(P).items():
        if not (name.startswith("test_") and callable(fn)):
            continue
        if name == "test_golden_closed_forms":
            calls += [(f"{name}[{c['name']}]", lambda c=c: P.test_golden_closed_forms(c)) for c in cases]
        elif name == "test_gradients_finite_differences":
            calls += [(f"{name}{a}", lambda a=a: P.test_gradients_finite_differences(*a))
                      for a in [(1.0, False, False), (0.73, True, False), (1.9, False, True)]]
        elif name == "test_temperature_gradients_finite_differences":
            calls += [(f"{name}[{t}]", lambda t=t: P.test_temperature_gradients_finite_differences(t))
                      for t in (2.0, 0.6)]
        else:
            calls.append((name, fn))
    return calls


def _module_from(src: str) -> types.ModuleType:
    mod = types.ModuleType("kl_oracle_under_test")
    exec(compile(src, "kl_oracle_under_test", "exec"), mod.__dict__)
    return mod


def _failing_pins(mod, stop_at_first: bool, pins=P, attr="O", calls=_pin_calls) -> list:
    real = getattr(pins, attr)
    setattr(pins, attr, mod)
    failed = []
    try:
        for name, call in calls():
            try:
                call()
            except Exception:  # an assertion, or a shape error the mistake causes
                failed.append(name)
                if stop_at_first:
                    break
    finally:
        setattr(pins, attr, real)
    return failed


def test_unchanged_source_passes_every_pin_through_this_harness():
    src = open(SRC).read()
    assert _failing_pins(_module_from(src), stop_at_first=False) == []


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_fails_a_pin(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"the oracle no longer holds: {old}"
    failed = _failing_pins(_module_from(src.replace(old, new)), stop_at_first=True)
    assert failed, f"no pin catches: {name}"


def test_unchanged_cache_oracle_passes_every_pin_through_this_harness():
    src = open(SRC_TOPK).read()
    assert _failing_pins(_module_from(src), False, PT, "T", _topk_pin_calls) == []


@pytest.mark.parametrize("name,old,new", MUTATIONS_TOPK, ids=[m[0] for m in MUTATIONS_TOPK])
def test_cache_oracle_mutation_fails_a_pin(name, old, new):
    src = open(SRC_TOPK).read()
    assert src.count(old) == 1, f"the cache oracle no longer holds: {old}"
    failed = _failing_pins(_module_from(src.replace(old, new)), True, PT, "T", _topk_pin_calls)
    assert failed, f"no pin catches: {name}"
