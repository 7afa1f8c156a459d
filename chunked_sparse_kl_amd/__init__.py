"""Python binding of kdloss, the fused chunked sparse-KL loss head for MI355X.

Thin ctypes layer over the C ABI declared in include/kdloss.h: the functions
below carry the same names as the C entry points and only marshal arguments
(torch tensors -> device pointers, the current HIP stream, a workspace tensor
sized by the planner).  Every step of the computation runs in the library's
HIP kernels; there is no fallback.  The library is loaded on the first call,
which raises if it has not been built (``python -m chunked_sparse_kl_amd.build``).

``fused_chunked_kl`` wraps forward and backward in an ``autograd.Function``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "KD_BF16", "KD_F32", "KdError", "kd_plan_query", "kd_fused_chunked_kl_fwd",
    "kd_fused_chunked_kl_bwd", "kd_set_validate", "kd_profile_enable", "kd_profile_reset",
    "kd_profile_read", "fused_chunked_kl", "library_path", "EXPORTED_SYMBOLS", "lib",
    "kd_teacher_topk_plan", "kd_teacher_topk", "kd_fused_chunked_kl_fwd_noalloc",
    "KD_NOALLOC_SCRATCH_BYTES", "KD_VARIANT_DENSE", "KD_VARIANT_FORWARD_CHUNKED",
    "kd_comparator_grid_bytes", "kd_dense_kl_fwd", "kd_dense_kl_bwd", "kd_forward_chunked_kl_fwd",
    "kd_forward_chunked_kl_bwd",
]

KD_BF16 = 0
KD_F32 = 1
_STATUS = {0: "KD_OK", -1: "KD_E_INVAL", -2: "KD_E_WORKSPACE", -3: "KD_E_HIP", -4: "KD_E_RANGE"}

EXPORTED_SYMBOLS = (
    "kd_plan_query", "kd_fused_chunked_kl_fwd", "kd_fused_chunked_kl_bwd", "kd_status_string",
    "kd_last_error_message", "kd_set_validate", "kd_profile_enable", "kd_profile_reset",
    "kd_profile_read",
    "kd_teacher_topk_plan", "kd_teacher_topk", "kd_fused_chunked_kl_fwd_noalloc",
    "kd_comparator_grid_bytes", "kd_dense_kl_fwd", "kd_dense_kl_bwd", "kd_forward_chunked_kl_fwd",
    "kd_forward_chunked_kl_bwd",
)

KD_VARIANT_DENSE = 1
KD_VARIANT_FORWARD_CHUNKED = 2

KD_NOALLOC_SCRATCH_BYTES = 256 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.environ.get("KDLOSS_LIBRARY", os.path.join(_HERE, "libkdloss.so"))


class KdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class KdPlan(ctypes.Structure):
    _fields_ = [
        ("chunk", ctypes.c_int64), ("n_chunks", ctypes.c_int64), ("vocab_tiles", ctypes.c_int64),
        ("dh_splits", ctypes.c_int64), ("fwd_workspace_bytes", ctypes.c_size_t),
        ("bwd_workspace_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t),
    ]


class KdTopkPlan(ctypes.Structure):
    _fields_ = [
        ("chunk", ctypes.c_int64), ("n_chunks", ctypes.c_int64), ("cap", ctypes.c_int64),
        ("vocab_tiles", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
    ]


class KdKernelStat(ctypes.Structure):
    _fields_ = [
        ("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
        ("flops", ctypes.c_double), ("bytes", ctypes.c_double),
    ]


def _load():
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"kdloss library not found at {path}; build it with "
                          f"`python -m chunked_sparse_kl_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.kd_plan_query.argtypes = [ctypes.c_int, i64, i64, i64, i32, i64, sz, ctypes.POINTER(KdPlan)]
    f32 = ctypes.c_float
    lib.kd_fused_chunked_kl_fwd.argtypes = [
        ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i64, i32, i64, f32, vp, sz, vp, vp, vp, vp, vp]
    lib.kd_fused_chunked_kl_bwd.argtypes = [
        ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i64, i32, i64, f32, vp, vp, vp, vp, ctypes.c_int,
        vp, sz, vp]
    lib.kd_fused_chunked_kl_fwd_noalloc.argtypes = [
        ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i64, i32, i64, f32, vp, vp, vp, vp, vp]
    cmp_fwd = [ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i64, i32, i64, vp, sz, vp, sz, vp, vp, vp, vp]
    cmp_bwd = [ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i64, i32, i64, vp, sz, vp, vp, vp, vp, ctypes.c_int,
               vp, sz, vp]
    lib.kd_comparator_grid_bytes.argtypes = [ctypes.c_int, i64, i64]
    lib.kd_comparator_grid_bytes.restype = sz
    for f in ("kd_dense_kl_fwd", "kd_forward_chunked_kl_fwd"):
        getattr(lib, f).argtypes = cmp_fwd
        getattr(lib, f).restype = ctypes.c_int
    for f in ("kd_dense_kl_bwd", "kd_forward_chunked_kl_bwd"):
        getattr(lib, f).argtypes = cmp_bwd
        getattr(lib, f).restype = ctypes.c_int
    lib.kd_status_string.argtypes = [ctypes.c_int]
    lib.kd_status_string.restype = ctypes.c_char_p
    lib.kd_last_error_message.argtypes = []
    lib.kd_last_error_message.restype = ctypes.c_char_p
    lib.kd_set_validate.argtypes = [ctypes.c_int]
    lib.kd_profile_enable.argtypes = [ctypes.c_int]
    lib.kd_profile_reset.argtypes = []
    lib.kd_profile_read.argtypes = [ctypes.POINTER(KdKernelStat), ctypes.c_int]
    lib.kd_teacher_topk_plan.argtypes = [ctypes.c_int, i64, i64, i64, i32, i64, i64, sz,
                                         ctypes.POINTER(KdTopkPlan)]
    lib.kd_teacher_topk.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, i32, i64, i64, vp, sz, vp, vp, vp]
    for f in ("kd_plan_query", "kd_fused_chunked_kl_fwd", "kd_fused_chunked_kl_fwd_noalloc",
              "kd_fused_chunked_kl_bwd",
              "kd_set_validate", "kd_profile_enable", "kd_profile_reset", "kd_profile_read",
              "kd_teacher_topk_plan", "kd_teacher_topk"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


_lib_handle = None


def lib():
    """The loaded ctypes library (loaded once; raises ImportError if not built)."""
    global _lib_handle
    if _lib_handle is None:
        _lib_handle = _load()
    return _lib_handle


def _check(rc: int) -> int:
    if rc < 0:
        raise KdError(rc, lib().kd_last_error_message().decode())
    return rc


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KD_BF16
    if t.dtype == torch.float32:
        return KD_F32
    raise TypeError(f"H and W must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_inputs(H, W, topk_idx, topk_logp, mask):
    if not (H.is_cuda and W.is_cuda and topk_idx.is_cuda and topk_logp.is_cuda):
        raise ValueError("H, W, topk_idx and topk_logp must be device tensors")
    if H.dtype != W.dtype:
        raise TypeError("H and W must share one dtype")
    for name, t in (("H", H), ("W", W), ("topk_idx", topk_idx), ("topk_logp", topk_logp)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if topk_idx.dtype != torch.int32 or topk_logp.dtype != torch.float32:
        raise TypeError("topk_idx must be int32 and topk_logp float32")
    if mask is not None and (mask.dtype != torch.uint8 or not mask.is_contiguous() or not mask.is_cuda):
        raise TypeError("mask must be a contiguous uint8 device tensor")
    n, d = H.shape
    V = W.shape[0]
    K = topk_idx.shape[1]
    if W.shape[1] != d or topk_idx.shape[0] != n or tuple(topk_logp.shape) != (n, K):
        raise ValueError("shape mismatch between H [n,d], W [V,d], topk_idx/topk_logp [n,K]")
    if mask is not None and mask.numel() != n:
        raise ValueError("mask must have n entries")
    return n, d, V, K


def kd_plan_query(dtype: int, n: int, d: int, V: int, K: int, chunk: int = 0,
                  hbm_budget: int = 0) -> dict:
    """Planner result as a dict (see kd_plan_query in include/kdloss.h)."""
    out = KdPlan()
    _check(lib().kd_plan_query(dtype, n, d, V, K, chunk, hbm_budget, ctypes.byref(out)))
    return {f: getattr(out, f) for f, _ in KdPlan._fields_}


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace too small: {nbytes} bytes needed")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def kd_fused_chunked_kl_fwd(H, W, topk_idx, topk_logp, mask=None, chunk: int = 0, workspace=None,
                            row_kl: bool = True, gathered: bool = False, plan: dict | None = None,
                            temperature: float = 1.0):
    """Forward call.  Returns a dict with loss [1], lse [n], row_kl [n] (optional),
    gathered [n, K] (optional) and the plan used.  ``temperature`` softens both
    sides and scales the loss by its square; ids < 0 in ``topk_idx`` are padding."""
    n, d, V, K = _check_inputs(H, W, topk_idx, topk_logp, mask)
    dt = _dtype_code(H)
    plan = plan or kd_plan_query(dt, n, d, V, K, chunk)
    ws = _workspace(plan["fwd_workspace_bytes"], H.device, workspace)
    loss = torch.empty(1, dtype=torch.float32, device=H.device)
    lse = torch.empty(n, dtype=torch.float32, device=H.device)
    rk = torch.empty(n, dtype=torch.float32, device=H.device) if row_kl else None
    g = torch.empty((n, K), dtype=torch.float32, device=H.device) if gathered else None
    _check(lib().kd_fused_chunked_kl_fwd(
        dt, _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logp), _ptr(mask), n, d, V, K,
        plan["chunk"], float(temperature), _ptr(ws), ws.numel() * ws.element_size(), _ptr(loss),
        _ptr(lse), _ptr(rk), _ptr(g), _stream(H.device)))
    return {"loss": loss, "lse": lse, "row_kl": rk, "gathered": g, "plan": plan}


def kd_fused_chunked_kl_fwd_noalloc(H, W, topk_idx, topk_logp, mask=None, chunk: int = 0,
                                    temperature: float = 1.0, loss=None, lse=None, row_kl=None,
                                    gathered=None):
    """Forward call that allocates nothing on the device: the library's
    per-GPU scratch array (KD_NOALLOC_SCRATCH_BYTES) is its workspace.  The
    outputs may be passed in (loss [1], lse [n], row_kl [n] or None, gathered
    [n, K] or None, fp32 device tensors); the ones left as None that are
    required (loss, lse) are allocated here, by torch, before the call.
    Returns a dict like kd_fused_chunked_kl_fwd's (without a plan).  Calls
    that overlap on one GPU share the scratch and must be serialised."""
    n, d, V, K = _check_inputs(H, W, topk_idx, topk_logp, mask)
    dt = _dtype_code(H)
    if loss is None:
        loss = torch.empty(1, dtype=torch.float32, device=H.device)
    if lse is None:
        lse = torch.empty(n, dtype=torch.float32, device=H.device)
    for name, t, shape in (("loss", loss, (1,)), ("lse", lse, (n,)), ("row_kl", row_kl, (n,)),
                           ("gathered", gathered, (n, K))):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shape
                              or not t.is_contiguous() or t.device != H.device):
            raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor on H's device")
    _check(lib().kd_fused_chunked_kl_fwd_noalloc(
        dt, _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logp), _ptr(mask), n, d, V, K, chunk,
        float(temperature), _ptr(loss), _ptr(lse), _ptr(row_kl), _ptr(gathered), _stream(H.device)))
    return {"loss": loss, "lse": lse, "row_kl": row_kl, "gathered": gathered}


def kd_fused_chunked_kl_bwd(H, W, topk_idx, topk_logp, mask, lse, grad_loss=None, chunk: int = 0,
                            workspace=None, dW=None, plan: dict | None = None, accumulate: bool = True,
                            temperature: float = 1.0):
    """Backward call.  Returns (dH, dW).  A given dW is accumulated into
    (accumulate=True) or overwritten (accumulate=False); without one, a new
    dW is allocated and written.  ``temperature`` must be the forward call's."""
    n, d, V, K = _check_inputs(H, W, topk_idx, topk_logp, mask)
    dt = _dtype_code(H)
    plan = plan or kd_plan_query(dt, n, d, V, K, chunk)
    ws = _workspace(plan["bwd_workspace_bytes"], H.device, workspace)
    if grad_loss is None:
        grad_loss = torch.ones(1, dtype=torch.float32, device=H.device)
    grad_loss = grad_loss.reshape(1).to(torch.float32).contiguous()
    dH = torch.empty_like(H)
    if dW is None:
        dW = torch.empty((V, d), dtype=torch.float32, device=H.device)
        accumulate = False
    elif dW.dtype != torch.float32 or tuple(dW.shape) != (V, d) or not dW.is_contiguous():
        raise ValueError("dW must be a contiguous float32 [V, d] tensor")
    _check(lib().kd_fused_chunked_kl_bwd(
        dt, _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logp), _ptr(mask), n, d, V, K,
        plan["chunk"], float(temperature), _ptr(lse), _ptr(grad_loss), _ptr(dH), _ptr(dW),
        1 if accumulate else 0,
        _ptr(ws), ws.numel() * ws.element_size(), _stream(H.device)))
    return dH, dW


def kd_comparator_grid_bytes(variant: int, n: int, V: int) -> int:
    """Bytes of the grid buffer a comparison variant keeps (KD_VARIANT_DENSE:
    log q and the teacher grid; KD_VARIANT_FORWARD_CHUNKED: the logits)."""
    nb = lib().kd_comparator_grid_bytes(variant, n, V)
    if nb == 0:
        raise ValueError(f"bad comparator arguments: variant={variant} n={n} V={V}")
    return nb


_CMP = {KD_VARIANT_DENSE: ("kd_dense_kl_fwd", "kd_dense_kl_bwd"),
        KD_VARIANT_FORWARD_CHUNKED: ("kd_forward_chunked_kl_fwd", "kd_forward_chunked_kl_bwd")}


def _comparator_fwd(variant, H, W, topk_idx, topk_logp, mask, chunk, workspace, grid, row_kl, plan):
    n, d, V, K = _check_inputs(H, W, topk_idx, topk_logp, mask)
    dt = _dtype_code(H)
    plan = plan or kd_plan_query(dt, n, d, V, K, chunk)
    ws = _workspace(plan["fwd_workspace_bytes"], H.device, workspace)
    gb = kd_comparator_grid_bytes(variant, n, V)
    grid = _workspace(gb, H.device, grid)
    loss = torch.empty(1, dtype=torch.float32, device=H.device)
    lse = torch.empty(n, dtype=torch.float32, device=H.device)
    rk = torch.empty(n, dtype=torch.float32, device=H.device) if row_kl else None
    _check(getattr(lib(), _CMP[variant][0])(
        dt, _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logp), _ptr(mask), n, d, V, K, plan["chunk"],
        _ptr(grid), grid.numel() * grid.element_size(), _ptr(ws), ws.numel() * ws.element_size(),
        _ptr(loss), _ptr(lse), _ptr(rk), _stream(H.device)))
    return {"loss": loss, "lse": lse, "row_kl": rk, "grid": grid, "plan": plan}


def _comparator_bwd(variant, H, W, topk_idx, topk_logp, mask, lse, grid, grad_loss, chunk, workspace, dW,
                    plan, accumulate):
    n, d, V, K = _check_inputs(H, W, topk_idx, topk_logp, mask)
    dt = _dtype_code(H)
    plan = plan or kd_plan_query(dt, n, d, V, K, chunk)
    ws = _workspace(plan["bwd_workspace_bytes"], H.device, workspace)
    if grad_loss is None:
        grad_loss = torch.ones(1, dtype=torch.float32, device=H.device)
    grad_loss = grad_loss.reshape(1).to(torch.float32).contiguous()
    dH = torch.empty_like(H)
    if dW is None:
        dW = torch.empty((V, d), dtype=torch.float32, device=H.device)
        accumulate = False
    elif dW.dtype != torch.float32 or tuple(dW.shape) != (V, d) or not dW.is_contiguous():
        raise ValueError("dW must be a contiguous float32 [V, d] tensor")
    _check(getattr(lib(), _CMP[variant][1])(
        dt, _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logp), _ptr(mask), n, d, V, K, plan["chunk"],
        _ptr(grid), grid.numel() * grid.element_size(), _ptr(lse), _ptr(grad_loss), _ptr(dH), _ptr(dW),
        1 if accumulate else 0, _ptr(ws), ws.numel() * ws.element_size(), _stream(H.device)))
    return dH, dW


def kd_dense_kl_fwd(H, W, topk_idx, topk_logp, mask=None, chunk: int = 0, workspace=None, grid=None,
                    row_kl: bool = True, plan: dict | None = None):
    """Dense-KL forward (comparison variant): builds the full log q and teacher
    grids in ``grid`` (allocated if not given) and returns loss, lse, row_kl,
    grid and plan.  The backward needs the same grid, unchanged."""
    return _comparator_fwd(KD_VARIANT_DENSE, H, W, topk_idx, topk_logp, mask, chunk, workspace, grid,
                           row_kl, plan)


def kd_dense_kl_bwd(H, W, topk_idx, topk_logp, mask, lse, grid, grad_loss=None, chunk: int = 0,
                    workspace=None, dW=None, plan: dict | None = None, accumulate: bool = True):
    """Dense-KL backward from the forward's grids: (dH, dW) as kd_fused_chunked_kl_bwd."""
    return _comparator_bwd(KD_VARIANT_DENSE, H, W, topk_idx, topk_logp, mask, lse, grid, grad_loss, chunk,
                           workspace, dW, plan, accumulate)


def kd_forward_chunked_kl_fwd(H, W, topk_idx, topk_logp, mask=None, chunk: int = 0, workspace=None,
                              grid=None, row_kl: bool = True, plan: dict | None = None):
    """Forward-chunked KL forward (comparison variant): the loss chunk by chunk
    with the logits of every chunk kept in ``grid`` for the backward."""
    return _comparator_fwd(KD_VARIANT_FORWARD_CHUNKED, H, W, topk_idx, topk_logp, mask, chunk, workspace,
                           grid, row_kl, plan)


def kd_forward_chunked_kl_bwd(H, W, topk_idx, topk_logp, mask, lse, grid, grad_loss=None, chunk: int = 0,
                              workspace=None, dW=None, plan: dict | None = None, accumulate: bool = True):
    """Forward-chunked KL backward from the kept logits: (dH, dW)."""
    return _comparator_bwd(KD_VARIANT_FORWARD_CHUNKED, H, W, topk_idx, topk_logp, mask, lse, grid, grad_loss,
                           chunk, workspace, dW, plan, accumulate)


def kd_teacher_topk_plan(dtype: int, n: int, d: int, V: int, K: int, chunk: int = 0, cap: int = 0,
                         hbm_budget: int = 0) -> dict:
    """Plan of the teacher top-K cache builder (see kd_teacher_topk_plan in include/kdloss.h)."""
    out = KdTopkPlan()
    _check(lib().kd_teacher_topk_plan(dtype, n, d, V, K, chunk, cap, hbm_budget, ctypes.byref(out)))
    return {f: getattr(out, f) for f, _ in KdTopkPlan._fields_}


def kd_teacher_topk(Ht, Wt, K: int, chunk: int = 0, cap: int = 0, workspace=None,
                    plan: dict | None = None):
    """Teacher top-K cache of the rows of Ht: (topk_idx [n, K] int32, topk_logp [n, K] fp32),
    ids in decreasing order of the logit Ht . Wt[v], values the full-vocabulary
    log-probabilities.  Synchronises the current stream (an offline step)."""
    if not (Ht.is_cuda and Wt.is_cuda):
        raise ValueError("Ht and Wt must be device tensors")
    if Ht.dtype != Wt.dtype:
        raise TypeError("Ht and Wt must share one dtype")
    if not (Ht.is_contiguous() and Wt.is_contiguous()):
        raise ValueError("Ht and Wt must be contiguous")
    n, d = Ht.shape
    V = Wt.shape[0]
    if Wt.shape[1] != d:
        raise ValueError("shape mismatch between Ht [n, d] and Wt [V, d]")
    dt = _dtype_code(Ht)
    plan = plan or kd_teacher_topk_plan(dt, n, d, V, K, chunk, cap)
    ws = _workspace(plan["workspace_bytes"], Ht.device, workspace)
    idx = torch.empty((n, K), dtype=torch.int32, device=Ht.device)
    logp = torch.empty((n, K), dtype=torch.float32, device=Ht.device)
    _check(lib().kd_teacher_topk(dt, _ptr(Ht), _ptr(Wt), n, d, V, K, plan["chunk"], plan["cap"], _ptr(ws),
                                 ws.numel() * ws.element_size(), _ptr(idx), _ptr(logp),
                                 _stream(Ht.device)))
    return idx, logp


def kd_set_validate(on: bool) -> None:
    _check(lib().kd_set_validate(1 if on else 0))


def kd_profile_enable(on: bool) -> None:
    _check(lib().kd_profile_enable(1 if on else 0))


def kd_profile_reset() -> None:
    _check(lib().kd_profile_reset())


def kd_profile_read() -> list[dict]:
    n = _check(lib().kd_profile_read(None, 0))
    arr = (KdKernelStat * max(n, 1))()
    m = _check(lib().kd_profile_read(arr, n))
    return [{"name": arr[i].name.decode(), "launches": arr[i].launches, "total_ms": arr[i].total_ms,
             "flops": arr[i].flops, "bytes": arr[i].bytes} for i in range(m)]


class _FusedChunkedKL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, W, topk_idx, topk_logp, mask, chunk, temperature):
        out = kd_fused_chunked_kl_fwd(H, W, topk_idx, topk_logp, mask, chunk, row_kl=False,
                                      temperature=temperature)
        ctx.save_for_backward(H, W, topk_idx, topk_logp, mask, out["lse"])
        ctx.plan = out["plan"]
        ctx.temperature = temperature
        return out["loss"][0]

    @staticmethod
    def backward(ctx, grad):
        H, W, topk_idx, topk_logp, mask, lse = ctx.saved_tensors
        dH, dW = kd_fused_chunked_kl_bwd(H, W, topk_idx, topk_logp, mask, lse,
                                         grad.reshape(1), plan=ctx.plan,
                                         temperature=ctx.temperature)
        return dH, dW.to(W.dtype), None, None, None, None, None


def fused_chunked_kl(H, W, topk_idx, topk_logp, mask=None, chunk: int = 0, temperature: float = 1.0):
    """Mean KL(teacher top-K renormalised || student full softmax) over unmasked rows,
    differentiable w.r.t. H and W.  With a temperature tau both distributions
    are softened by it and the loss is multiplied by tau^2."""
    return _FusedChunkedKL.apply(H, W, topk_idx, topk_logp, mask, chunk, float(temperature))
