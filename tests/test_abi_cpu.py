"""Host-side checks of the C ABI: the library loads, exports what include/kdloss.h
declares, the planner behaves as documented, and bad arguments are rejected
before any device work (no kernel is launched in these tests)."""
import ctypes
import os
import re
import subprocess

import pytest

import chunked_sparse_kl_amd as kd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdloss.h")
GiB = 1 << 30


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(kd.library_path()):
        from chunked_sparse_kl_amd import build
        build.build()
    return kd.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kd_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert _declared_functions() == sorted(kd.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", kd.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b[TW] (kd_[a-z_]+)$", out, flags=re.M))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(kd.lib(), name)


def test_status_strings():
    lib = kd.lib()
    for code, name in [(0, b"KD_OK"), (-1, b"KD_E_INVAL"), (-2, b"KD_E_WORKSPACE"), (-3, b"KD_E_HIP"),
                       (-4, b"KD_E_RANGE")]:
        assert lib.kd_status_string(code) == name


@pytest.mark.parametrize("n,d,V,want", [
    (4096, 3072, 128256, 2048),      # toy head, 4K tokens
    (8192, 3072, 128256, 4096),      # packed 8K
    (32768, 2880, 201088, 8192),     # 32K, large vocabulary
    (262144, 3072, 128256, 8192),    # 256K
    (256, 256, 4096, 256),           # small: a single chunk
    (300, 256, 4096, 256),
])
def test_planner_default_chunks(n, d, V, want):
    p = kd.kd_plan_query(kd.KD_BF16, n, d, V, 100, 0, 200 * GiB)
    assert p["chunk"] == want
    assert p["n_chunks"] == -(-n // want)
    assert p["workspace_bytes"] == max(p["fwd_workspace_bytes"], p["bwd_workspace_bytes"])


def test_planner_respects_budget_and_explicit_chunk():
    big = kd.kd_plan_query(kd.KD_BF16, 32768, 2880, 201088, 100, 0, 200 * GiB)
    small = kd.kd_plan_query(kd.KD_BF16, 32768, 2880, 201088, 100, 0, big["workspace_bytes"] // 3)
    assert small["chunk"] < big["chunk"] and small["chunk"] % 256 == 0
    assert small["workspace_bytes"] <= big["workspace_bytes"] // 3
    # a buffer of exactly the planned size yields the same plan (fwd/bwd use that rule)
    same = kd.kd_plan_query(kd.KD_BF16, 32768, 2880, 201088, 100, 0, big["workspace_bytes"])
    assert same == big
    expl = kd.kd_plan_query(kd.KD_F32, 256, 256, 4096, 16, 64, 0)
    assert expl["chunk"] == 64 and expl["n_chunks"] == 4
    with pytest.raises(kd.KdError) as e:
        kd.kd_plan_query(kd.KD_BF16, 32768, 2880, 201088, 100, 0, 1 << 20)
    assert e.value.status == -2


def test_workspace_is_linear_in_rows():
    # fixed chunk: every buffer other than the per-chunk ones scales with n
    sizes = [kd.kd_plan_query(kd.KD_BF16, n, 3072, 128256, 100, 8192, 0)["workspace_bytes"]
             for n in (16384, 32768, 65536, 131072, 262144)]
    slopes = [(b - a) / (m - k) for a, b, k, m in zip(sizes, sizes[1:], (16384, 32768, 65536, 131072),
                                                        (32768, 65536, 131072, 262144))]
    assert max(slopes) - min(slopes) <= 0.01 * max(slopes)
    assert max(slopes) < 4096  # bytes per row: teacher buffers only, never a vocabulary-sized row


@pytest.mark.parametrize("kwargs,code", [
    (dict(dtype=2), -1), (dict(n=0), -1), (dict(K=5000), -1), (dict(d=250), -1), (dict(chunk=100), -1),
])
def test_bad_sizes_rejected(kwargs, code):
    args = dict(dtype=kd.KD_BF16, n=1000, d=256, V=4096, K=16, chunk=0)
    args.update(kwargs)
    with pytest.raises(kd.KdError) as e:
        kd.kd_plan_query(args["dtype"], args["n"], args["d"], args["V"], args["K"], args["chunk"], GiB)
    assert e.value.status == code


def test_null_pointers_rejected_without_device_work():
    lib = kd.lib()
    loss = ctypes.c_void_p(16)
    rc = lib.kd_fused_chunked_kl_fwd(0, None, None, None, None, None, 256, 256, 4096, 16, 64, 1.0, None,
                                     0, loss, loss, None, None, None)
    assert rc == -1 and b"non-null" in lib.kd_last_error_message()
    fake = ctypes.c_void_p(4096)
    rc = lib.kd_fused_chunked_kl_fwd(0, fake, fake, fake, fake, None, 256, 256, 4096, 16, 64, 1.0, None,
                                     0, fake, fake, None, None, None)
    assert rc == -2 and b"workspace" in lib.kd_last_error_message()
    misaligned = ctypes.c_void_p(4104)
    rc = lib.kd_fused_chunked_kl_bwd(0, misaligned, fake, fake, fake, None, 256, 256, 4096, 16, 64,
                                     1.0, fake, fake, fake, fake, 1, fake, 1 << 30, None)
    assert rc == -1 and b"aligned" in lib.kd_last_error_message()


@pytest.mark.parametrize("tau", [0.0, -1.0, float("nan"), float("inf")])
def test_bad_temperature_rejected_without_device_work(tau):
    lib = kd.lib()
    fake = ctypes.c_void_p(4096)
    rc = lib.kd_fused_chunked_kl_fwd(0, fake, fake, fake, fake, None, 256, 256, 4096, 16, 64, tau, fake,
                                     1 << 30, fake, fake, None, None, None)
    assert rc == -1 and b"temperature" in lib.kd_last_error_message()
    rc = lib.kd_fused_chunked_kl_bwd(0, fake, fake, fake, fake, None, 256, 256, 4096, 16, 64, tau, fake,
                                     fake, fake, fake, 1, fake, 1 << 30, None)
    assert rc == -1 and b"temperature" in lib.kd_last_error_message()


# ------------------------------------------------------------------ teacher top-K cache builder
def test_topk_plan_defaults():
    p = kd.kd_teacher_topk_plan(kd.KD_BF16, 32768, 2880, 201088, 100, 0, 0, GiB * 8)
    assert p["cap"] == 4096 and p["vocab_tiles"] == 786 and p["chunk"] % 256 == 0
    assert p["workspace_bytes"] <= GiB * 8
    # fewer 256-wide tiles than K: every logit is a candidate
    p = kd.kd_teacher_topk_plan(kd.KD_F32, 700, 192, 1100, 24, 256, 0, GiB)
    assert p["cap"] == 1100 and p["chunk"] == 256 and p["n_chunks"] == 3
    p = kd.kd_teacher_topk_plan(kd.KD_F32, 700, 192, 8000, 24, 0, 100, GiB)
    assert p["cap"] == 100


@pytest.mark.parametrize("kwargs", [dict(K=5000), dict(cap=10), dict(chunk=100), dict(V=10), dict(d=250)])
def test_topk_plan_rejects(kwargs):
    args = dict(dtype=kd.KD_BF16, n=1000, d=256, V=8000, K=24, chunk=0, cap=0)
    args.update(kwargs)
    with pytest.raises(kd.KdError) as e:
        kd.kd_teacher_topk_plan(args["dtype"], args["n"], args["d"], args["V"], args["K"], args["chunk"],
                                args["cap"], GiB)
    assert e.value.status == -1


def test_topk_null_pointers_and_small_workspace_rejected_without_device_work():
    lib = kd.lib()
    fake = ctypes.c_void_p(4096)
    rc = lib.kd_teacher_topk(0, None, fake, 256, 256, 4096, 16, 64, 0, fake, 1 << 30, fake, fake, None)
    assert rc == -1 and b"non-null" in lib.kd_last_error_message()
    rc = lib.kd_teacher_topk(0, fake, fake, 256, 256, 4096, 16, 64, 0, fake, 16, fake, fake, None)
    assert rc == -2 and b"workspace" in lib.kd_last_error_message()


@pytest.mark.parametrize("n,d,V,K", [(32768, 2880, 201088, 100), (4096, 3072, 128256, 100), (200, 256, 4096, 16)])
def test_auto_chunk_calls_plan_against_their_own_workspace(n, d, V, K):
    """chunk <= 0 with a buffer of the planner's per-call size: the forward
    needs only plan.fwd_workspace_bytes and the backward plan.bwd_workspace_bytes.
    A null loss / lse pointer is the next check after planning, so reaching
    it (KD_E_INVAL, "non-null") shows the plan fitted; no device work is done."""
    lib = kd.lib()
    p = kd.kd_plan_query(kd.KD_BF16, n, d, V, K, 0, 200 * GiB)
    fake = ctypes.c_void_p(4096)
    rc = lib.kd_fused_chunked_kl_fwd(0, fake, fake, fake, fake, None, n, d, V, K, 0, 1.0, fake,
                                     p["fwd_workspace_bytes"], None, fake, None, None, None)
    assert rc == -1 and b"non-null" in lib.kd_last_error_message(), lib.kd_last_error_message()
    rc = lib.kd_fused_chunked_kl_bwd(0, fake, fake, fake, fake, None, n, d, V, K, 0, 1.0, None, fake,
                                     fake, fake, 0, fake, p["bwd_workspace_bytes"], None)
    assert rc == -1 and b"non-null" in lib.kd_last_error_message(), lib.kd_last_error_message()
    # one byte less than the smallest plan of that call is still reported as a workspace shortfall
    small = kd.kd_plan_query(kd.KD_BF16, n, d, V, K, min(256, n), 200 * GiB)
    rc = lib.kd_fused_chunked_kl_fwd(0, fake, fake, fake, fake, None, n, d, V, K, 0, 1.0, fake,
                                     small["fwd_workspace_bytes"] - 1, None, fake, None, None, None)
    assert rc == -2 and b"bytes" in lib.kd_last_error_message()


def test_comparator_grid_bytes_and_refusals_without_device_work():
    lib = kd.lib()
    n, V = 32768, 201088
    one = n * (-(-V // 64) * 64) * 4
    assert kd.kd_comparator_grid_bytes(kd.KD_VARIANT_DENSE, n, V) == 2 * one
    assert kd.kd_comparator_grid_bytes(kd.KD_VARIANT_FORWARD_CHUNKED, n, V) == one
    assert lib.kd_comparator_grid_bytes(3, n, V) == 0 and lib.kd_comparator_grid_bytes(1, 0, V) == 0
    fake = ctypes.c_void_p(4096)
    p = kd.kd_plan_query(kd.KD_BF16, 256, 256, 4096, 16, 64, 0)
    for fwd in (lib.kd_dense_kl_fwd, lib.kd_forward_chunked_kl_fwd):
        # a grid one byte short
        need = lib.kd_comparator_grid_bytes(1 if fwd is lib.kd_dense_kl_fwd else 2, 256, 4096)
        rc = fwd(0, fake, fake, fake, fake, None, 256, 256, 4096, 16, 64, fake, need - 1, fake,
                 p["fwd_workspace_bytes"], fake, fake, None, None)
        assert rc == -2 and b"grid" in lib.kd_last_error_message()
        # fp32 inputs
        rc = fwd(1, fake, fake, fake, fake, None, 256, 256, 4096, 16, 64, fake, need, fake,
                 p["fwd_workspace_bytes"], fake, fake, None, None)
        assert rc == -1 and b"bf16" in lib.kd_last_error_message()
    for bwd in (lib.kd_dense_kl_bwd, lib.kd_forward_chunked_kl_bwd):
        rc = bwd(0, fake, fake, fake, fake, None, 256, 256, 4096, 16, 64, None, 0, fake, fake, fake, fake, 0,
                 fake, p["bwd_workspace_bytes"], None)
        assert rc == -2 and b"grid" in lib.kd_last_error_message()
