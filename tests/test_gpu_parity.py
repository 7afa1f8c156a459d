"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle.

Small cases are compared element by element over every row; they are sized
to span several 256-row / 256-vocabulary tiles, a ragged vocabulary tile, a
ragged K (hidden-dim) block and a ragged last chunk.  The five workloads are
checked at full size on a seeded row subset (per-row values on the subset in
the run as given; loss, dH and dW in a second run whose mask keeps only the
subset), in the chunking the benchmark uses.
"""
import numpy as np
import pytest
import torch

import chunked_sparse_kl_amd as kd
from chunked_sparse_kl_amd import synth
from oracle import kl_oracle as O
from tests.parity_util import check_full, check_subset, rel_fro, run_gpu

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _name(request):
    _log(f"[case] {request.node.name}")
    yield


# ------------------------------------------------------------------ small, full comparison
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("chunk", [256, 448, 0])
def test_small_ragged(dtype, chunk):
    inp = synth.make_custom(700, 200, 1000, 20, dtype, "random5", "uniform", seed=11)
    gpu = run_gpu(inp, chunk=chunk)
    check_full(inp, gpu, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [320, 288])
def test_narrow_last_column_tile(dtype, d):
    # d = 256 + 64 / 256 + 32: the dH and dW tiles of the last 256 hidden
    # columns hold only 64 / 32 valid columns; 4 chunks, so dW is written by
    # the first pair and accumulated by the second
    inp = synth.make_custom(700, d, 1100, 24, dtype, "random5", "uniform", seed=25)
    gpu = run_gpu(inp, chunk=192, grad=1.3)
    assert gpu["plan"]["n_chunks"] == 4
    check_full(inp, gpu, dtype, grad=1.3)


@pytest.mark.parametrize("dtype,n,d,V,K", [("bf16", 70, 40, 100, 7), ("f32", 33, 12, 50, 50),
                                           ("bf16", 5, 8, 300, 3)])
def test_below_one_tile_and_one_k_block(dtype, n, d, V, K):
    # d below one 64-wide K block (only the ragged block runs), V below or just
    # over one 256-wide vocabulary tile, n below one 256-row tile
    inp = synth.make_custom(n, d, V, K, dtype, "random5", "uniform", seed=26)
    gpu = run_gpu(inp, chunk=0)
    check_full(inp, gpu, dtype)


def test_tiny_fp32_workload_full():
    inp = synth.make_inputs(1)
    gpu = run_gpu(inp, chunk=inp["workload"].chunk)
    assert gpu["plan"]["chunk"] == 64
    check_full(inp, gpu, "f32")


@pytest.mark.parametrize("n", [1, 63, 65])
def test_few_rows(n):
    inp = synth.make_custom(n, 64, 777, 5, "bf16", "ones", "uniform", seed=3)
    check_full(inp, run_gpu(inp), "bf16")


def test_k_equals_v_and_k_one():
    inp = synth.make_custom(96, 64, 320, 320, "bf16", "random5", "uniform", seed=4)
    check_full(inp, run_gpu(inp, chunk=64), "bf16")
    inp = synth.make_custom(96, 64, 320, 1, "bf16", "random5", "uniform", seed=5)
    check_full(inp, run_gpu(inp, chunk=64), "bf16")


def test_duplicates_neginf_and_shifted_teacher():
    inp = synth.make_custom(300, 128, 900, 12, "bf16", "random5", "uniform", seed=6)
    inp["idx"][3, 1] = inp["idx"][3, 0]            # duplicate id within a row: summed
    inp["idx"][7, 2:5] = inp["idx"][7, 1]
    inp["logp"][10, -1] = float("-inf")            # zero-probability entry
    inp["logp"] += torch.randn(300, 1) * 5.0       # raw logits, not log-probs: renormalised over K
    gpu = run_gpu(inp, chunk=128, grad=0.37)
    check_full(inp, gpu, "bf16", grad=0.37)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_register_and_general_teacher_paths_agree(dtype):
    """Rows of K <= 128 entries are prepared from registers, longer rows by the
    general loop.  The same rows at K = 100 and padded to K = 140 (ids -1 at
    the end, garbage log-values under them) take one path each and give
    bit-identical results: padding adds exact zeros, repeated ids are summed
    in k order on both paths."""
    inp = synth.make_custom(700, 128, 1500, 100, dtype, "random5", "uniform", seed=31)
    idx = inp["idx"].numpy()
    rng = np.random.default_rng(31)
    for t in range(0, 700, 5):
        src = rng.choice(100, size=6, replace=False)
        dst = rng.choice(100, size=6, replace=False)
        idx[t, dst] = idx[t, src]
    idx[2, 60:70] = idx[2, 0]                      # across the 64-entry boundary
    inp["idx"] = torch.from_numpy(idx)
    padded = dict(inp)
    padded["idx"] = torch.cat([inp["idx"], torch.full((700, 40), -1, dtype=torch.int32)], 1).contiguous()
    padded["logp"] = torch.cat([inp["logp"], torch.full((700, 40), 3.0)], 1).contiguous()
    a = run_gpu(inp, chunk=192, grad=0.9)
    b = run_gpu(padded, chunk=192, grad=0.9)
    assert a["loss"] == b["loss"]
    for k in ("lse", "row_kl", "dH", "dW"):
        assert np.array_equal(a[k], b[k]), k
    live = inp["mask"].numpy() != 0
    assert np.array_equal(a["g"][live], b["g"][live][:, :100])
    check_full(inp, a, dtype, grad=0.9)


@pytest.mark.parametrize("K", [63, 64, 65, 127, 128, 129])
def test_teacher_row_lengths_at_the_lane_boundaries(K):
    """K around one and two 64-lane rows of entries: 64 and 128 fill the
    registers of the register path exactly, 65 puts one entry in the second
    register, 129 takes the general path.  Rows repeat ids across the two
    registers."""
    inp = synth.make_custom(200, 64, 2000, K, "bf16", "random5", "uniform", seed=32 + K)
    idx = inp["idx"].numpy()
    idx[1, K - 1] = idx[1, 0]
    idx[3, K // 2:K // 2 + 3] = idx[3, 1]
    inp["idx"] = torch.from_numpy(idx)
    inp["mask"][[1, 3]] = 1
    check_full(inp, run_gpu(inp, chunk=128, grad=1.3), "bf16", grad=1.3)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_negative_incoming_gradient(dtype):
    """grad_loss < 0: the gradients are the negated ones of |grad_loss|.  bf16 G
    carries the sign of the row factor apart from its magnitude, so G itself is
    exactly negated; the bf16 MFMA's fp32 accumulation is not exactly symmetric
    under negation of an operand (about 8% of dW's fp32 entries move by an
    ulp, measured), so dH and dW are compared bit for bit in fp32 and to a
    relative 1e-6 in bf16."""
    inp = synth.make_custom(400, 96, 1300, 24, dtype, "random5", "uniform", seed=33)
    idx = inp["idx"].numpy()
    idx[5, 3] = idx[5, 0]                          # a repeated id
    inp["idx"] = torch.from_numpy(idx)
    inp["mask"][5] = 1
    pos = run_gpu(inp, chunk=192, grad=0.8)
    neg = run_gpu(inp, chunk=192, grad=-0.8)
    assert neg["loss"] == pos["loss"]
    if dtype == "f32":
        assert np.array_equal(neg["dH"], -pos["dH"]) and np.array_equal(neg["dW"], -pos["dW"])
    assert rel_fro(neg["dH"], -pos["dH"]) <= 1e-6 and rel_fro(neg["dW"], -pos["dW"]) <= 1e-6
    check_full(inp, neg, dtype, grad=-0.8)


def test_clustered_ids_overflow_tiles():
    # every teacher id of every row inside one 256-wide vocabulary tile
    inp = synth.make_custom(256, 64, 2048, 100, "bf16", "ones", "uniform", seed=8)
    rng = np.random.default_rng(0)
    inp["idx"] = torch.from_numpy(np.stack([rng.permutation(256)[:100] + 512 for _ in range(256)]).astype(np.int32))
    check_full(inp, run_gpu(inp, chunk=128), "bf16")


# ------------------------------------------------------------------ temperature, padding
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("tau", [2.0, 0.5])
def test_temperature(dtype, tau):
    inp = synth.make_custom(600, 192, 1100, 24, dtype, "random5", "uniform", seed=21)
    inp["logp"] += torch.randn(600, 1) * 3.0       # any per-row offset
    gpu = run_gpu(inp, chunk=256, grad=0.8, temperature=tau)
    check_full(inp, gpu, dtype, grad=0.8, temperature=tau)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_padding_entries(dtype):
    inp = synth.make_custom(500, 128, 900, 16, dtype, "random5", "uniform", seed=22)
    rng = np.random.default_rng(22)
    n_real = rng.integers(1, 17, size=500)         # rows hold 1..16 real entries, the rest padding
    idx = inp["idx"].numpy()
    for t in range(500):
        idx[t, n_real[t]:] = -1 - rng.integers(0, 5, size=16 - n_real[t])
    inp["logp"][torch.from_numpy(idx < 0)] = 7.0   # padding log-values are ignored
    inp["idx"] = torch.from_numpy(idx)
    gpu = run_gpu(inp, chunk=128, temperature=1.5)
    check_full(inp, gpu, dtype, temperature=1.5)


def test_padding_equals_shorter_teacher_rows():
    # padding at the end of every row == the same rows with K reduced
    inp = synth.make_custom(300, 64, 700, 12, "bf16", "random5", "uniform", seed=23)
    short = dict(inp)
    short["idx"] = inp["idx"][:, :8].contiguous()
    short["logp"] = inp["logp"][:, :8].contiguous()
    padded = dict(inp)
    padded["idx"] = inp["idx"].clone()
    padded["idx"][:, 8:] = -1
    a = run_gpu(short, chunk=128, gathered=False)
    b = run_gpu(padded, chunk=128, gathered=False)
    assert abs(a["loss"] - b["loss"]) <= 1e-6 * abs(a["loss"])
    np.testing.assert_allclose(b["row_kl"], a["row_kl"], rtol=1e-5, atol=1e-6)
    assert np.array_equal(a["lse"], b["lse"])
    assert rel_fro(b["dH"], a["dH"]) <= 1e-2 and rel_fro(b["dW"], a["dW"]) <= 1e-5


def test_bad_temperature_is_an_error():
    inp = synth.make_custom(64, 64, 300, 4, "bf16", "ones", "uniform", seed=24)
    with pytest.raises(kd.KdError):
        run_gpu(inp, temperature=0.0)


# ------------------------------------------------------------------ semantics
def test_all_masked_rows_give_zero():
    inp = synth.make_custom(200, 64, 500, 8, "bf16", "ones", "uniform", seed=9)
    inp["mask"][:] = 0
    gpu = run_gpu(inp, chunk=64)
    assert gpu["loss"] == 0.0
    assert not gpu["dH"].any() and not gpu["dW"].any()
    assert np.isfinite(gpu["lse"]).all()


def test_masked_rows_never_read():
    inp = synth.make_custom(256, 64, 700, 10, "bf16", "random5", "uniform", seed=10)
    clean = run_gpu(inp, chunk=64)
    dead = inp["mask"] == 0
    inp["logp"][dead] = float("nan")
    inp["idx"][dead] = -77777
    dirty = run_gpu(inp, chunk=64)
    assert dirty["loss"] == clean["loss"]
    assert np.array_equal(dirty["dW"], clean["dW"]) and np.array_equal(dirty["dH"], clean["dH"])


def test_chunk_size_independence_bitwise_loss():
    inp = synth.make_custom(1000, 256, 3000, 16, "bf16", "random5", "uniform", seed=12)
    ref = run_gpu(inp, chunk=1000)
    live = inp["mask"].numpy() != 0  # gathered values are undefined on masked rows
    for c in (64, 192, 256, 512, 0):
        got = run_gpu(inp, chunk=c)
        assert got["loss"] == ref["loss"], c
        assert np.array_equal(got["lse"], ref["lse"]) and np.array_equal(got["row_kl"], ref["row_kl"])
        assert np.array_equal(got["g"][live], ref["g"][live])
        assert rel_fro(got["dW"], ref["dW"]) <= 1e-5 and rel_fro(got["dH"], ref["dH"]) <= 5e-3


def test_deterministic_repeat():
    inp = synth.make_custom(600, 256, 2000, 16, "bf16", "random5", "uniform", seed=13)
    a = run_gpu(inp, chunk=256)
    b = run_gpu(inp, chunk=256)
    assert a["loss"] == b["loss"]
    for k in ("lse", "row_kl", "g", "dH", "dW"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_deterministic_repeat_with_duplicate_ids(dtype):
    # K = 100 (two 64-lane chunks per row): rows repeat ids within and across
    # the chunks, two and three times, several rows share a vocabulary tile
    inp = synth.make_custom(640, 192, 1500, 100, dtype, "random5", "uniform", seed=27)
    idx = inp["idx"].numpy()
    rng = np.random.default_rng(27)
    for t in range(0, 640, 3):
        src = rng.choice(100, size=12, replace=False)
        dst = rng.choice(100, size=12, replace=False)
        idx[t, dst] = idx[t, src]
    idx[1, 70:] = idx[1, :30]                      # across the 64-entry boundary
    idx[2, [0, 64, 99]] = idx[2, 5]                # three occurrences
    idx[4, :] = idx[4, 7]                          # one id, 100 times
    idx[5, :] = np.tile(idx[5, :5], 20)            # five ids, 20 times each
    idx[6, ::2] = -1                               # padding between repeats
    idx[6, 1::4] = idx[6, 3]
    inp["idx"] = torch.from_numpy(idx)
    inp["mask"][[4, 5, 6]] = 1
    runs = [run_gpu(inp, chunk=128, grad=0.6) for _ in range(3)]
    for r in runs[1:]:
        assert r["loss"] == runs[0]["loss"]
        for k in ("lse", "row_kl", "g", "dH", "dW"):
            assert np.array_equal(r[k], runs[0][k]), k
    check_full(inp, runs[0], dtype, grad=0.6)


@pytest.mark.parametrize("chunk", [520, 192, 128])
def test_dw_overwrite_mode(chunk):
    """accumulate=False never reads dW (NaN-filled here) and matches a fresh
    result bit for bit; so does accumulating onto zeros.  192 and 128 give 3
    and 5 chunks: the G^T pairs end on a lone chunk."""
    inp = synth.make_custom(520, 64, 1100, 12, "bf16", "random5", "uniform", seed=15)
    d = {k: v.cuda() for k, v in inp.items() if torch.is_tensor(v)}
    fw = kd.kd_fused_chunked_kl_fwd(d["H"], d["W"], d["idx"], d["logp"], d["mask"], chunk=chunk)
    args = (d["H"], d["W"], d["idx"], d["logp"], d["mask"], fw["lse"])
    _, dw_new = kd.kd_fused_chunked_kl_bwd(*args, plan=fw["plan"])
    nan = torch.full_like(dw_new, float("nan"))
    _, dw_over = kd.kd_fused_chunked_kl_bwd(*args, dW=nan, plan=fw["plan"], accumulate=False)
    zero = torch.zeros_like(dw_new)
    _, dw_acc = kd.kd_fused_chunked_kl_bwd(*args, dW=zero, plan=fw["plan"], accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dw_new, dw_over) and torch.equal(dw_new, dw_acc)
    b = O.backward(inp["H"], inp["W"], inp["idx"].numpy(), inp["logp"], inp["mask"].numpy())
    assert rel_fro(dw_new.cpu().double().numpy(), b["dW"]) <= 1e-2


@pytest.mark.parametrize("chunk", [300, 128])
def test_dw_accumulates_and_grad_scales(chunk):
    inp = synth.make_custom(300, 64, 900, 12, "bf16", "random5", "uniform", seed=14)
    d = {k: v.cuda() for k, v in inp.items() if torch.is_tensor(v)}
    fw = kd.kd_fused_chunked_kl_fwd(d["H"], d["W"], d["idx"], d["logp"], d["mask"], chunk=chunk)
    g = torch.tensor([0.5], device="cuda")
    dH1, dW = kd.kd_fused_chunked_kl_bwd(d["H"], d["W"], d["idx"], d["logp"], d["mask"], fw["lse"], g, plan=fw["plan"])
    dW1 = dW.clone()
    dH2, dW = kd.kd_fused_chunked_kl_bwd(d["H"], d["W"], d["idx"], d["logp"], d["mask"], fw["lse"], g,
                                         dW=dW, plan=fw["plan"])
    torch.cuda.synchronize()
    assert torch.equal(dH1, dH2)
    if chunk >= 300:  # one chunk: 0 + a, then a + a, both exact
        assert torch.equal(dW, dW1 * 2)
    else:             # several chunks: the second call adds chunk by chunk onto dW1
        assert rel_fro(dW.cpu().double().numpy(), 2 * dW1.cpu().double().numpy()) <= 1e-6
    b = O.backward(inp["H"], inp["W"], inp["idx"].numpy(), inp["logp"], inp["mask"].numpy(), grad_loss=0.5)
    assert rel_fro(dW1.cpu().double().numpy(), b["dW"]) <= 1e-2


def test_validation_reports_out_of_range_ids():
    inp = synth.make_custom(128, 64, 500, 8, "bf16", "ones", "uniform", seed=15)
    inp["idx"][5, 3] = 500
    d = {k: v.cuda() for k, v in inp.items() if torch.is_tensor(v)}
    kd.kd_set_validate(True)
    try:
        with pytest.raises(kd.KdError) as e:
            kd.kd_fused_chunked_kl_fwd(d["H"], d["W"], d["idx"], d["logp"], d["mask"], chunk=64)
        assert e.value.status == -4
    finally:
        kd.kd_set_validate(False)
    # without validation the id is skipped, nothing is read out of range
    out = kd.kd_fused_chunked_kl_fwd(d["H"], d["W"], d["idx"], d["logp"], d["mask"], chunk=64)
    torch.cuda.synchronize()
    assert np.isfinite(out["loss"].item())


def test_autograd_function():
    inp = synth.make_custom(320, 128, 1100, 10, "bf16", "random5", "uniform", seed=16)
    d = {k: v.cuda() for k, v in inp.items() if torch.is_tensor(v)}
    H = d["H"].clone().requires_grad_(True)
    W = d["W"].clone().requires_grad_(True)
    loss = kd.fused_chunked_kl(H, W, d["idx"], d["logp"], d["mask"], chunk=128) * 2.0
    loss.backward()
    b = O.backward(inp["H"], inp["W"], inp["idx"].numpy(), inp["logp"], inp["mask"].numpy(), grad_loss=2.0)
    assert rel_fro(H.grad.float().cpu().double().numpy(), b["dH"]) <= 1e-2
    assert rel_fro(W.grad.float().cpu().double().numpy(), b["dW"]) <= 1e-2


# ------------------------------------------------------------------ gather, bit exact
@pytest.mark.parametrize("T,d,V,K,chunk", [(700, 64, 1000, 20, 256), (32768, 2880, 201088, 100, 0)])
def test_gather_integer_encoded_exact(T, d, V, K, chunk):
    # W[v, 0:3] = base-256 digits of v, H[t, 0:3] = (65536, 256, 1): every logit
    # z_{t,v} = v exactly in bf16 x bf16 -> fp32, so the gathered value must equal the id.
    inp = synth.make_custom(T, d, V, K, "bf16", "random5", "uniform", seed=17)
    v = torch.arange(V)
    W = torch.zeros(V, d)
    W[:, 0], W[:, 1], W[:, 2] = (v // 65536).float(), ((v // 256) % 256).float(), (v % 256).float()
    H = torch.zeros(T, d)
    H[:, 0], H[:, 1], H[:, 2] = 65536.0, 256.0, 1.0
    inp["W"], inp["H"] = W.to(torch.bfloat16), H.to(torch.bfloat16)
    gpu = run_gpu(inp, chunk=chunk)
    live = inp["mask"].numpy() != 0
    assert np.array_equal(gpu["g"][live], inp["idx"].numpy()[live].astype(np.float64))


# ------------------------------------------------------------------ the five workloads
def test_workload1_tiny_fp32():
    inp = synth.make_inputs(1)
    gpu = run_gpu(inp, chunk=64)
    check_full(inp, gpu, "f32")


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_workload_subset(cfg):
    inp = synth.make_inputs(cfg)
    _log(f"  generated inputs for workload {cfg}")
    res = check_subset(inp, chunk=0, dtype="bf16")
    _log(f"  workload {cfg}: {res}")
