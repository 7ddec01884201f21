"""Python binding of libfljsd (the C ABI in include/fljsd.h).

Argument marshalling only: tensors become device pointers, the current HIP
stream is passed through, status codes become exceptions. Every step of the
pass runs in the library's HIP kernels; there is no fallback. PyTorch provides
device memory and streams.

The library must be built first (``python -m lm_head_distillation_amd.build``).
torch is imported before the library is loaded so the library binds to the
HIP runtime torch already loaded (both carry the soname libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfljsd.so")

F32, BF16 = 0, 1
REDUCTIONS = {"batchmean": 0, "sum": 1, "mean": 2, "none": 3}
STATUS = {0: "FLJSD_OK", -1: "FLJSD_EINVAL", -2: "FLJSD_EDTYPE", -3: "FLJSD_EWORKSPACE",
          -4: "FLJSD_EALIGN", -5: "FLJSD_EHIP", -6: "FLJSD_EDEVICE"}
KERNEL_CLASSES = ["gemm_logits", "jsd_stats", "jsd_loss", "jsd_grad", "gemm_grad_input",
                  "splitk_reduce", "gemm_grad_weight", "loss_reduce", "transpose", "elem_loss", "ce_stats", "ce_grad"]

_lib = None


class FljsdError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libfljsd.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing; build it with "
                          "`python -m lm_head_distillation_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, sz, vp, f32, cint = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    lib.fljsd_forward_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, cint, f32, f32,
                                           cint, cint, vp, vp, vp, vp, sz, vp]
    lib.fljsd_forward_backward.restype = cint
    lib.fljsd_forward_backward_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, cint, f32, f32,
                                              cint, cint, vp, vp, vp, cint, ctypes.c_uint, vp, sz,
                                              vp]
    lib.fljsd_forward_backward_ex.restype = cint
    lib.fljsd_generalized_jsd.argtypes = [vp, vp, i64, i64, i64, cint, f32, f32, cint, vp, vp,
                                          vp, sz, vp]
    lib.fljsd_generalized_jsd.restype = cint
    lib.fljsd_generalized_jsd_noalloc.argtypes = [vp, vp, i64, i64, i64, cint, f32, f32, cint,
                                                  vp, vp, vp]
    lib.fljsd_generalized_jsd_noalloc.restype = cint
    lib.fljsd_jsd_logprob.argtypes = [vp, vp, i64, i64, i64, cint, f32, cint, vp, vp, vp, sz, vp]
    lib.fljsd_jsd_logprob.restype = cint
    lib.fljsd_tvd.argtypes = [vp, vp, i64, i64, i64, cint, cint, vp, vp, vp, sz, vp]
    lib.fljsd_tvd.restype = cint
    lib.fljsd_flce_forward_backward.argtypes = [vp, vp, vp, i64, i64, i64, cint, i64, f32, cint, cint,
                                                vp, vp, vp, vp, sz, vp]
    lib.fljsd_flce_forward_backward.restype = cint
    lib.fljsd_flce_forward_backward_ex.argtypes = [vp, vp, vp, i64, i64, i64, cint, i64, f32, cint,
                                                   cint, vp, vp, vp, cint, ctypes.c_uint, vp, sz, vp]
    lib.fljsd_flce_forward_backward_ex.restype = cint
    lib.fljsd_flce_workspace_size.argtypes = [i64, i64, i64, cint, cint]
    lib.fljsd_flce_workspace_size.restype = sz
    lib.fljsd_flce_plan_num_chunks.argtypes = [i64, i64, i64, cint, sz]
    lib.fljsd_flce_plan_num_chunks.restype = cint
    lib.fljsd_workspace_size.argtypes = [i64, i64, i64, i64, cint, cint]
    lib.fljsd_workspace_size.restype = sz
    lib.fljsd_generalized_jsd_workspace_size.argtypes = [i64, i64, cint]
    lib.fljsd_generalized_jsd_workspace_size.restype = sz
    lib.fljsd_plan_num_chunks.argtypes = [i64, i64, i64, i64, cint, sz]
    lib.fljsd_plan_num_chunks.restype = cint
    lib.fljsd_strerror.argtypes = [cint]
    lib.fljsd_strerror.restype = ctypes.c_char_p
    lib.fljsd_last_error.argtypes = []
    lib.fljsd_last_error.restype = ctypes.c_char_p
    lib.fljsd_profile_enable.argtypes = [cint]
    lib.fljsd_profile_enable.restype = cint
    lib.fljsd_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), cint]
    lib.fljsd_profile_read.restype = cint
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != 0:
        lib = load_library()
        raise FljsdError(rc, f"{lib.fljsd_strerror(rc).decode()} ({lib.fljsd_last_error().decode()})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _reduction_code(reduction: str) -> int:
    try:
        return REDUCTIONS[reduction]
    except KeyError:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}") from None


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check_out(t: torch.Tensor, dtype: torch.dtype, numel: int, device, what: str) -> None:
    """A caller-supplied output: its dtype, element count, device and layout
    must be what the library writes, or the kernels would write past it."""
    if t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{what} must hold {numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{what} must live on {device}")


def _check_workspace(ws: torch.Tensor, device) -> None:
    if not ws.is_cuda or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")


def _require_device(*tensors: torch.Tensor) -> None:
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("tensors must live in GPU memory")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.device != tensors[0].device:
            raise ValueError("tensors must live on one device")


def fljsd_workspace_size(BT: int, H_s: int, H_t: int, V: int, dtype: int, num_chunks: int) -> int:
    return int(load_library().fljsd_workspace_size(BT, H_s, H_t, V, dtype, num_chunks))


def fljsd_generalized_jsd_workspace_size(BT: int, V: int, dtype: int) -> int:
    return int(load_library().fljsd_generalized_jsd_workspace_size(BT, V, dtype))


def fljsd_plan_num_chunks(BT: int, H_s: int, H_t: int, V: int, dtype: int, budget_bytes: int) -> int:
    rc = load_library().fljsd_plan_num_chunks(BT, H_s, H_t, V, dtype, budget_bytes)
    if rc < 0:
        _check(rc)
    return int(rc)


def default_budget_bytes() -> int:
    """Workspace budget for the chunk policy: FLJSD_HBM_BUDGET_BYTES, else half
    of the device memory free right now."""
    env = os.environ.get("FLJSD_HBM_BUDGET_BYTES")
    if env:
        return int(env)
    free, _total = torch.cuda.mem_get_info()
    return free // 2


FLJSD_ACCUMULATE_GRAD_W = 1
FLJSD_TEMPERATURE_SQUARED = 2


def fljsd_forward_backward(X_s: torch.Tensor, W_s: torch.Tensor, X_t: torch.Tensor,
                           W_t: torch.Tensor, beta: float, temperature: float,
                           reduction: str = "batchmean", num_chunks: int = 0, *,
                           grad_input: bool = True, grad_weight: bool = True,
                           workspace: Optional[torch.Tensor] = None,
                           out: Optional[Tuple[torch.Tensor, Optional[torch.Tensor], Optional[torch.Tensor]]] = None,
                           stream=None):
    """Fused-linear JSD forward + backward. Returns (loss, grad_X_s, grad_W_s).

    num_chunks = 0 lets the policy pick the chunk count for the workspace
    budget (the given workspace's size, else default_budget_bytes()).
    Gradients not asked for are returned as None.
    """
    return fljsd_forward_backward_ex(X_s, W_s, X_t, W_t, beta, temperature, reduction,
                                     num_chunks, grad_w_dtype=None, flags=0,
                                     grad_input=grad_input, grad_weight=grad_weight,
                                     workspace=workspace, out=out, stream=stream, _entry="plain")


def fljsd_forward_backward_ex(X_s: torch.Tensor, W_s: torch.Tensor, X_t: torch.Tensor,
                              W_t: torch.Tensor, beta: float, temperature: float,
                              reduction: str = "batchmean", num_chunks: int = 0, *,
                              grad_w_dtype: Optional[torch.dtype] = None, flags: int = 0,
                              grad_input: bool = True, grad_weight: bool = True,
                              workspace: Optional[torch.Tensor] = None,
                              out: Optional[Tuple[torch.Tensor, Optional[torch.Tensor], Optional[torch.Tensor]]] = None,
                              stream=None, _entry: str = "ex"):
    """fljsd_forward_backward with a weight-gradient dtype and flags.

    grad_w_dtype: None (the input dtype) or torch.float32 (fp32 accumulation
    over chunks for bf16 inputs). flags: 0 or FLJSD_ACCUMULATE_GRAD_W, which
    adds to the grad_W_s given in ``out`` instead of overwriting it.
    """
    lib = load_library()
    _require_device(X_s, W_s, X_t, W_t)
    dt = _dtype_code(X_s)
    for t in (W_s, X_t, W_t):
        if _dtype_code(t) != dt:
            raise ValueError("all inputs must share one dtype")
    BT, H_s = X_s.shape
    V = W_s.shape[0]
    H_t = X_t.shape[1]
    if W_s.shape != (V, H_s) or X_t.shape != (BT, H_t) or W_t.shape != (V, H_t):
        raise ValueError("shape mismatch: X_s [BT,H_s], W_s [V,H_s], X_t [BT,H_t], W_t [V,H_t]")
    red = _reduction_code(reduction)
    gw_torch = X_s.dtype if grad_w_dtype is None else grad_w_dtype
    gw_code = {torch.float32: 0, torch.bfloat16: 1}.get(gw_torch, -1)
    if (flags & FLJSD_ACCUMULATE_GRAD_W) and (out is None or out[2] is None):
        raise ValueError("FLJSD_ACCUMULATE_GRAD_W needs the grad_W_s to add to, passed in `out`")
    nc = int(num_chunks)
    if nc == 0:
        budget = workspace.numel() * workspace.element_size() if workspace is not None else default_budget_bytes()
        nc = fljsd_plan_num_chunks(BT, H_s, H_t, V, dt, budget)
    need = fljsd_workspace_size(BT, H_s, H_t, V, dt, nc)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=X_s.device)
    if workspace is not None:
        _check_workspace(workspace, X_s.device)
    if out is not None:
        loss, gX, gW = out
        _check_out(loss, torch.float32, BT if red == 3 else 1, X_s.device, "loss")
        if gX is not None:
            _check_out(gX, X_s.dtype, BT * H_s, X_s.device, "grad_X_s")
        if gW is not None:
            _check_out(gW, gw_torch, V * H_s, X_s.device, "grad_W_s")
    else:
        loss = torch.empty(BT if red == 3 else 1, dtype=torch.float32, device=X_s.device)
        gX = torch.empty_like(X_s) if grad_input else None
        gW = torch.empty(V, H_s, dtype=gw_torch, device=X_s.device) if grad_weight else None
    args = (X_s.data_ptr(), W_s.data_ptr(), X_t.data_ptr(), W_t.data_ptr(), BT, H_s, H_t, V, dt,
            float(beta), float(temperature), red, nc, loss.data_ptr(), _ptr(gX), _ptr(gW))
    tail = (workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream))
    if _entry == "plain":
        rc = lib.fljsd_forward_backward(*args, *tail)
    else:
        rc = lib.fljsd_forward_backward_ex(*args, gw_code, int(flags), *tail)
    _check(rc)
    return (loss if red == 3 else loss[0]), gX, gW


def fljsd_generalized_jsd(logits_s: torch.Tensor, logits_t: torch.Tensor, beta: float,
                          temperature: float, reduction: str = "batchmean", *,
                          grad: Optional[torch.Tensor] = None, in_place: bool = False,
                          want_grad: bool = True, workspace: Optional[torch.Tensor] = None,
                          stream=None):
    """Generalized JSD over given logits [BT, V] (rows may be padded: the row
    stride is taken from the tensor). Returns (loss, grad_logits_s or None).

    in_place=True writes the gradient over logits_s and returns it.
    """
    lib = load_library()
    for t in (logits_s, logits_t):
        if not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError("logits must be 2-D GPU tensors with unit column stride")
    dt = _dtype_code(logits_s)
    if _dtype_code(logits_t) != dt:
        raise ValueError("logits must share one dtype")
    BT, V = logits_s.shape
    ld = logits_s.stride(0)
    if logits_t.shape != (BT, V) or logits_t.stride(0) != ld:
        raise ValueError("logits_t must match logits_s in shape and row stride")
    if logits_t.device != logits_s.device:
        raise ValueError("logits must live on one device")
    red = _reduction_code(reduction)
    need = fljsd_generalized_jsd_workspace_size(BT, V, dt)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits_s.device)
    _check_workspace(workspace, logits_s.device)
    loss = torch.empty(BT if red == 3 else 1, dtype=torch.float32, device=logits_s.device)
    if in_place:
        grad = logits_s
    elif want_grad and grad is None:
        grad = torch.empty_strided(logits_s.shape, logits_s.stride(), dtype=logits_s.dtype,
                                   device=logits_s.device)
    elif not want_grad:
        grad = None
    if grad is not None and (grad.stride() != logits_s.stride() or grad.shape != logits_s.shape
                             or grad.dtype != logits_s.dtype or grad.device != logits_s.device):
        raise ValueError("grad must match logits_s in dtype, shape, strides and device")
    rc = lib.fljsd_generalized_jsd(
        logits_s.data_ptr(), logits_t.data_ptr(), BT, V, ld, dt, float(beta), float(temperature),
        red, loss.data_ptr(), _ptr(grad), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc)
    return (loss if red == 3 else loss[0]), grad


NOALLOC_SCRATCH_BYTES = 8 << 20


def fljsd_generalized_jsd_noalloc(logits_s: torch.Tensor, logits_t: torch.Tensor, beta: float,
                                  temperature: float, reduction: str = "batchmean", *,
                                  loss: torch.Tensor, grad: Optional[torch.Tensor] = None,
                                  stream=None):
    """fljsd_generalized_jsd through the entry point that allocates nothing:
    the caller passes the outputs (``loss``: 1 fp32 value, or BT for "none";
    ``grad`` shaped and strided like logits_s, may be logits_s itself, or None)
    and the library uses its per-GPU scratch array. Calls that overlap on one
    GPU race. Returns (loss, grad)."""
    lib = load_library()
    dt, BT, V, ld = _pair_2d(logits_s, logits_t, "logits")
    red = _reduction_code(reduction)
    _check_out(loss, torch.float32, BT if red == 3 else 1, logits_s.device, "loss")
    if grad is not None and (grad.dtype != logits_s.dtype or grad.shape != logits_s.shape
                             or grad.stride() != logits_s.stride() or grad.device != logits_s.device):
        raise ValueError("grad must match logits_s in dtype, shape, strides and device")
    rc = lib.fljsd_generalized_jsd_noalloc(
        logits_s.data_ptr(), logits_t.data_ptr(), BT, V, ld, dt, float(beta), float(temperature),
        red, loss.data_ptr(), _ptr(grad), _stream(stream))
    _check(rc)
    return loss, grad


def _pair_2d(a: torch.Tensor, b: torch.Tensor, what: str):
    for t in (a, b):
        if not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{what} must be 2-D GPU tensors with unit column stride")
    dt = _dtype_code(a)
    if _dtype_code(b) != dt:
        raise ValueError(f"{what} must share one dtype")
    BT, V = a.shape
    ld = a.stride(0)
    if b.shape != (BT, V) or b.stride(0) != ld:
        raise ValueError(f"{what}: second input must match the first in shape and row stride")
    if b.device != a.device:
        raise ValueError(f"{what} must live on one device")
    return dt, BT, V, ld


def _grad_like(a: torch.Tensor, grad, in_place: bool, want_grad: bool):
    if in_place:
        return a
    if not want_grad:
        return None
    if grad is None:
        grad = torch.empty_strided(a.shape, a.stride(), dtype=a.dtype, device=a.device)
    if (grad.stride() != a.stride() or grad.shape != a.shape or grad.dtype != a.dtype
            or grad.device != a.device):
        raise ValueError("grad must match the input in dtype, shape, strides and device")
    return grad


def fljsd_jsd_logprob(logq_s: torch.Tensor, logp_t: torch.Tensor, beta: float,
                      reduction: str = "batchmean", *, grad: Optional[torch.Tensor] = None,
                      in_place: bool = False, want_grad: bool = True,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Generalized JSD over given log-probabilities [BT, V]. Returns
    (loss, d loss / d logq_s or None)."""
    lib = load_library()
    dt, BT, V, ld = _pair_2d(logq_s, logp_t, "log-probabilities")
    red = _reduction_code(reduction)
    if workspace is None:
        workspace = torch.empty(fljsd_generalized_jsd_workspace_size(BT, V, dt), dtype=torch.uint8,
                                device=logq_s.device)
    _check_workspace(workspace, logq_s.device)
    loss = torch.empty(BT if red == 3 else 1, dtype=torch.float32, device=logq_s.device)
    grad = _grad_like(logq_s, grad, in_place, want_grad)
    rc = lib.fljsd_jsd_logprob(logq_s.data_ptr(), logp_t.data_ptr(), BT, V, ld, dt, float(beta), red,
                               loss.data_ptr(), _ptr(grad), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc)
    return (loss if red == 3 else loss[0]), grad


def fljsd_tvd(p: torch.Tensor, q: torch.Tensor, reduction: str = "batchmean", *,
              grad: Optional[torch.Tensor] = None, in_place: bool = False, want_grad: bool = True,
              workspace: Optional[torch.Tensor] = None, stream=None):
    """Total variation distance between distributions p, q [BT, V]. Returns
    (loss, d loss / d p or None); reduction "none" gives the [BT, V] losses."""
    lib = load_library()
    dt, BT, V, ld = _pair_2d(p, q, "distributions")
    red = _reduction_code(reduction)
    if workspace is None:
        workspace = torch.empty(fljsd_generalized_jsd_workspace_size(BT, V, dt), dtype=torch.uint8,
                                device=p.device)
    _check_workspace(workspace, p.device)
    loss = torch.empty((BT, V) if red == 3 else (1,), dtype=torch.float32, device=p.device)
    grad = _grad_like(p, grad, in_place, want_grad)
    rc = lib.fljsd_tvd(p.data_ptr(), q.data_ptr(), BT, V, ld, dt, red, loss.data_ptr(), _ptr(grad),
                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                       _stream(stream))
    _check(rc)
    return (loss if red == 3 else loss[0]), grad


def fljsd_flce_workspace_size(BT: int, H: int, V: int, dtype: int, num_chunks: int) -> int:
    return int(load_library().fljsd_flce_workspace_size(BT, H, V, dtype, num_chunks))


def fljsd_flce_plan_num_chunks(BT: int, H: int, V: int, dtype: int, budget_bytes: int) -> int:
    lib = load_library()
    rc = lib.fljsd_flce_plan_num_chunks(BT, H, V, dtype, budget_bytes)
    _check(rc if rc < 0 else 0)
    return rc


def fljsd_flce_forward_backward(X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
                                ignore_index: int = -100, label_smoothing: float = 0.0,
                                reduction: str = "mean", num_chunks: int = 0, *,
                                grad_input: bool = True, grad_weight: bool = True,
                                workspace: Optional[torch.Tensor] = None, stream=None):
    """Fused-linear cross-entropy forward + backward with hard labels.
    Returns (loss, grad_X or None, grad_W or None)."""
    return fljsd_flce_forward_backward_ex(X, W, labels, ignore_index, label_smoothing, reduction,
                                          num_chunks, grad_input=grad_input,
                                          grad_weight=grad_weight, workspace=workspace,
                                          stream=stream, _entry="plain")


def fljsd_flce_forward_backward_ex(X: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
                                   ignore_index: int = -100, label_smoothing: float = 0.0,
                                   reduction: str = "mean", num_chunks: int = 0, *,
                                   grad_w_dtype: Optional[torch.dtype] = None, flags: int = 0,
                                   grad_input: bool = True, grad_weight: bool = True,
                                   workspace: Optional[torch.Tensor] = None,
                                   out: Optional[Tuple[torch.Tensor, Optional[torch.Tensor], Optional[torch.Tensor]]] = None,
                                   stream=None, _entry: str = "ex"):
    """fljsd_flce_forward_backward with a weight-gradient dtype (None: the input
    dtype; torch.float32 with bf16 inputs: per-chunk products summed in fp32)
    and flags (FLJSD_ACCUMULATE_GRAD_W adds to the grad_W given in ``out``)."""
    lib = load_library()
    _require_device(X, W)
    dt = _dtype_code(X)
    if _dtype_code(W) != dt:
        raise ValueError("X and W must share one dtype")
    BT, H = X.shape
    V = W.shape[0]
    if W.shape != (V, H):
        raise ValueError("shape mismatch: X [BT,H], W [V,H]")
    if labels.dtype != torch.int64 or labels.shape != (BT,) or not labels.is_cuda or not labels.is_contiguous():
        raise ValueError("labels must be a contiguous int64 GPU tensor of shape [BT]")
    if labels.device != X.device:
        raise ValueError("labels must live on the inputs' device")
    red = _reduction_code(reduction)
    gw_torch = X.dtype if grad_w_dtype is None else grad_w_dtype
    gw_code = {torch.float32: 0, torch.bfloat16: 1}.get(gw_torch, -1)
    if (flags & FLJSD_ACCUMULATE_GRAD_W) and (out is None or out[2] is None):
        raise ValueError("FLJSD_ACCUMULATE_GRAD_W needs the grad_W to add to, passed in `out`")
    nc = int(num_chunks)
    if nc == 0:
        budget = workspace.numel() * workspace.element_size() if workspace is not None else default_budget_bytes()
        nc = fljsd_flce_plan_num_chunks(BT, H, V, dt, budget)
    if workspace is None:
        workspace = torch.empty(fljsd_flce_workspace_size(BT, H, V, dt, nc), dtype=torch.uint8,
                                device=X.device)
    _check_workspace(workspace, X.device)
    if out is not None:
        loss, gX, gW = out
        _check_out(loss, torch.float32, BT if red == 3 else 1, X.device, "loss")
        if gX is not None:
            _check_out(gX, X.dtype, BT * H, X.device, "grad_X")
        if gW is not None:
            _check_out(gW, gw_torch, V * H, X.device, "grad_W")
    else:
        loss = torch.empty(BT if red == 3 else 1, dtype=torch.float32, device=X.device)
        gX = torch.empty_like(X) if grad_input else None
        gW = torch.empty(V, H, dtype=gw_torch, device=X.device) if grad_weight else None
    args = (X.data_ptr(), W.data_ptr(), labels.data_ptr(), BT, H, V, dt, int(ignore_index),
            float(label_smoothing), red, nc, loss.data_ptr(), _ptr(gX), _ptr(gW))
    tail = (workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream))
    if _entry == "plain":
        rc = lib.fljsd_flce_forward_backward(*args, *tail)
    else:
        rc = lib.fljsd_flce_forward_backward_ex(*args, gw_code, int(flags), *tail)
    _check(rc)
    return (loss if red == 3 else loss[0]), gX, gW


def fljsd_profile_enable(enable: bool = True) -> None:
    _check(load_library().fljsd_profile_enable(1 if enable else 0))


def fljsd_profile_read() -> dict:
    """Per kernel class: total ms, launches, algorithmic flops and HBM bytes."""
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    launches = (ctypes.c_int64 * n)()
    flops = (ctypes.c_double * n)()
    nbytes = (ctypes.c_double * n)()
    _check(load_library().fljsd_profile_read(ms, launches, flops, nbytes, n))
    return {name: {"ms": ms[i], "launches": launches[i], "flops": flops[i], "bytes": nbytes[i]}
            for i, name in enumerate(KERNEL_CLASSES)}
