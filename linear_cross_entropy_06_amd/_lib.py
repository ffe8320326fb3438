"""ctypes binding of libflce.so (the C ABI declared in include/flce.h).

Argument marshalling only: tensors are checked for device, dtype and
layout, outputs are allocated with torch on the tensors' device, and raw
device pointers plus the current HIP stream are handed to the library.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  If the library is not built, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libflce.so")

FLCE_BF16 = 0
FLCE_F32 = 1

STATUS = {
    0: "FLCE_OK",
    1: "FLCE_ERR_INVALID_ARG",
    2: "FLCE_ERR_WORKSPACE",
    3: "FLCE_ERR_UNSUPPORTED",
    4: "FLCE_ERR_HIP",
    5: "FLCE_ERR_SCRATCH",
}

# Static device scratch of flce_fwd_bwd_noalloc (FLCE_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 512 << 20

# Every entry point include/flce.h declares.
EXPORTS = (
    "flce_workspace_bytes",
    "flce_fwd_bwd",
    "flce_fwd_bwd_accumulate",
    "flce_scale_grads",
    "flce_launch_count",
    "flce_fwd_bwd_timed",
    "flce_logits",
    "flce_ce_rows",
    "flce_cross_entropy",
    "flce_fwd_bwd_vocab",
    "flce_vocab_workspace_bytes",
    "flce_fwd_bwd_rmsnorm",
    "flce_rmsnorm_workspace_bytes",
    "flce_orpo_fwd_bwd",
    "flce_orpo_workspace_bytes",
    "flce_mfma_rate",
    "flce_fwd_bwd_noalloc",
    "flce_status_string",
)

FLCE_STEPS = 5
STEP_NAMES = ("logits_gemm", "ce_rows", "loss_sum", "grad_h_gemm", "grad_W_gemm")

_lib = None


class FlceError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load() -> ctypes.CDLL:
    """Load libflce.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m linear_cross_entropy_06_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.flce_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.flce_workspace_bytes.restype = sz
    lib.flce_fwd_bwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp, sz,
                                 ctypes.c_int, vp]
    lib.flce_fwd_bwd.restype = ctypes.c_int
    lib.flce_fwd_bwd_accumulate.argtypes = lib.flce_fwd_bwd.argtypes
    lib.flce_fwd_bwd_accumulate.restype = ctypes.c_int
    lib.flce_scale_grads.argtypes = [vp, i64, vp, i64, vp, ctypes.c_int, vp]
    lib.flce_scale_grads.restype = ctypes.c_int
    lib.flce_launch_count.argtypes = [i64, i64]
    lib.flce_launch_count.restype = i64
    lib.flce_fwd_bwd_timed.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp, sz,
                                       ctypes.c_int, vp, vp, i64]
    lib.flce_fwd_bwd_timed.restype = ctypes.c_int
    lib.flce_logits.argtypes = [vp, vp, i64, i64, i64, vp, i64, ctypes.c_int, vp]
    lib.flce_logits.restype = ctypes.c_int
    lib.flce_ce_rows.argtypes = [vp, i64, vp, i64, i64, ctypes.c_float, vp, i64,
                                 ctypes.c_int, vp]
    lib.flce_ce_rows.restype = ctypes.c_int
    lib.flce_cross_entropy.argtypes = [vp, i64, vp, i64, i64, vp, vp, ctypes.c_int, vp]
    lib.flce_cross_entropy.restype = ctypes.c_int
    lib.flce_fwd_bwd_vocab.argtypes = lib.flce_fwd_bwd.argtypes
    lib.flce_fwd_bwd_vocab.restype = ctypes.c_int
    lib.flce_vocab_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.flce_vocab_workspace_bytes.restype = sz
    lib.flce_fwd_bwd_rmsnorm.argtypes = [vp, vp, ctypes.c_float, vp, vp, i64, i64, i64, i64,
                                         vp, vp, vp, vp, vp, sz, ctypes.c_int, vp]
    lib.flce_fwd_bwd_rmsnorm.restype = ctypes.c_int
    lib.flce_rmsnorm_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.flce_rmsnorm_workspace_bytes.restype = sz
    lib.flce_orpo_fwd_bwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, vp,
                                      vp, vp, vp, vp, sz, ctypes.c_int, vp]
    lib.flce_orpo_fwd_bwd.restype = ctypes.c_int
    lib.flce_orpo_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int]
    lib.flce_orpo_workspace_bytes.restype = sz
    lib.flce_mfma_rate.argtypes = [vp, i64, i64, i64, vp, vp, vp]
    lib.flce_mfma_rate.restype = ctypes.c_int
    lib.flce_fwd_bwd_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, vp, vp,
                                         ctypes.c_int, vp]
    lib.flce_fwd_bwd_noalloc.restype = ctypes.c_int
    lib.flce_status_string.argtypes = [ctypes.c_int]
    lib.flce_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load().flce_status_string(status).decode()
        raise FlceError(status, msg)


def _dt(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return FLCE_BF16
    if x.dtype == torch.float32:
        return FLCE_F32
    raise TypeError(f"unsupported dtype {x.dtype}; expected bfloat16 or float32")


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need_cuda(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def workspace_bytes(N: int, H: int, V: int, chunk: int, dtype: torch.dtype) -> int:
    dt = FLCE_BF16 if dtype == torch.bfloat16 else FLCE_F32
    return int(load().flce_workspace_bytes(N, H, V, chunk, dt))


class HipEvents:
    """A host array of timing-enabled hipEvent_t handles (HIP runtime calls
    through ctypes), for flce_fwd_bwd_timed."""

    def __init__(self, n: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                  ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.n = n
        self.array = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.array[i] = h.value

    def elapsed_ms(self, i: int, j: int) -> float:
        out = ctypes.c_float()
        if self._hip.hipEventSynchronize(self.array[j]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        if self._hip.hipEventElapsedTime(ctypes.byref(out), self.array[i], self.array[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self) -> None:
        for i in range(self.n):
            if self.array[i]:
                self._hip.hipEventDestroy(self.array[i])
                self.array[i] = None


def launch_count(N: int, chunk: int) -> int:
    return int(load().flce_launch_count(N, chunk))


def fwd_bwd(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
            chunk: Optional[int] = None, *,
            loss: Optional[torch.Tensor] = None,
            grad_h: Optional[torch.Tensor] = None,
            grad_W: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None,
            events: Optional[HipEvents] = None,
            accumulate: bool = False,
            ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Mean cross-entropy loss of h W^T against targets, with dloss/dh and
    dloss/dW, via ``flce_fwd_bwd`` (or ``flce_fwd_bwd_timed`` when
    ``events`` is given, or ``flce_fwd_bwd_accumulate`` when ``accumulate``:
    dloss/dW is then added to the given fp32 ``grad_W``).  Returns (loss []
    fp32, grad_h like h, grad_W [V, H] fp32).  Buffers may be passed in to
    avoid allocation."""
    lib = load()
    _need_cuda(h, W, targets)
    if targets.dtype != torch.int32:
        raise TypeError("targets must be int32")
    if W.dtype != h.dtype:
        raise TypeError("h and W must share a dtype")
    N, H = h.shape
    V = W.shape[0]
    chunk = N if chunk is None else int(chunk)
    dt = _dt(h)
    dev = h.device
    if loss is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
    if grad_h is None:
        grad_h = torch.empty_like(h)
    if grad_W is None:
        if accumulate:
            raise ValueError("accumulate=True adds into a given grad_W")
        grad_W = torch.empty((V, H), dtype=torch.float32, device=dev)
    if accumulate and events is not None:
        raise ValueError("the timed entry point does not accumulate")
    need = int(lib.flce_workspace_bytes(N, H, V, chunk, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need_cuda(loss, grad_h, grad_W, workspace)
    args = (h.data_ptr(), W.data_ptr(), targets.data_ptr(), N, H, V, chunk,
            loss.data_ptr(), grad_h.data_ptr(), grad_W.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            dt, _stream_ptr(dev))
    if accumulate:
        st = lib.flce_fwd_bwd_accumulate(*args)
    elif events is None:
        st = lib.flce_fwd_bwd(*args)
    else:
        st = lib.flce_fwd_bwd_timed(*args, events.array, events.n)
    _check(st)
    return loss, grad_h, grad_W


def fwd_bwd_noalloc(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, chunk: int, *,
                    loss: torch.Tensor, grad_h: torch.Tensor, grad_W: torch.Tensor,
                    ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """``fwd_bwd`` through ``flce_fwd_bwd_noalloc``: no workspace argument,
    the library's static device scratch instead, and the outputs given by
    the caller (this function allocates nothing)."""
    lib = load()
    _need_cuda(h, W, targets, loss, grad_h, grad_W)
    if targets.dtype != torch.int32:
        raise TypeError("targets must be int32")
    if W.dtype != h.dtype:
        raise TypeError("h and W must share a dtype")
    N, H = h.shape
    V = W.shape[0]
    _check(lib.flce_fwd_bwd_noalloc(h.data_ptr(), W.data_ptr(), targets.data_ptr(), N, H, V,
                                    int(chunk), loss.data_ptr(), grad_h.data_ptr(),
                                    grad_W.data_ptr(), _dt(h), _stream_ptr(h.device)))
    return loss, grad_h, grad_W


def vocab_workspace_bytes(N: int, H: int, V: int, vchunk: int, dtype: torch.dtype) -> int:
    """Workspace of ``flce_fwd_bwd_vocab`` (0: shape not supported there)."""
    dt = FLCE_BF16 if dtype == torch.bfloat16 else FLCE_F32
    return int(load().flce_vocab_workspace_bytes(N, H, V, vchunk, dt))


def fwd_bwd_vocab(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, vchunk: int, *,
                  loss: Optional[torch.Tensor] = None,
                  grad_h: Optional[torch.Tensor] = None,
                  grad_W: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """The same outputs as ``fwd_bwd`` through ``flce_fwd_bwd_vocab``: all
    tokens at once, the vocabulary in column chunks of ``vchunk`` (logits
    formed twice; bf16 with H % 64 == 0, V % 64 == 0 and vchunk % 128 == 0
    or vchunk >= V)."""
    lib = load()
    _need_cuda(h, W, targets)
    if targets.dtype != torch.int32:
        raise TypeError("targets must be int32")
    if W.dtype != h.dtype:
        raise TypeError("h and W must share a dtype")
    N, H = h.shape
    V = W.shape[0]
    dt = _dt(h)
    dev = h.device
    if loss is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
    if grad_h is None:
        grad_h = torch.empty_like(h)
    if grad_W is None:
        grad_W = torch.empty((V, H), dtype=torch.float32, device=dev)
    need = int(lib.flce_vocab_workspace_bytes(N, H, V, int(vchunk), dt))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need_cuda(loss, grad_h, grad_W, workspace)
    st = lib.flce_fwd_bwd_vocab(h.data_ptr(), W.data_ptr(), targets.data_ptr(), N, H, V,
                                int(vchunk), loss.data_ptr(), grad_h.data_ptr(),
                                grad_W.data_ptr(), workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), dt,
                                _stream_ptr(dev))
    _check(st)
    return loss, grad_h, grad_W


def rmsnorm_workspace_bytes(N: int, H: int, V: int, chunk: int, dtype: torch.dtype) -> int:
    """Workspace of ``flce_fwd_bwd_rmsnorm``."""
    dt = FLCE_BF16 if dtype == torch.bfloat16 else FLCE_F32
    return int(load().flce_rmsnorm_workspace_bytes(N, H, V, chunk, dt))


def fwd_bwd_rmsnorm(x: torch.Tensor, gamma: torch.Tensor, W: torch.Tensor,
                    targets: torch.Tensor, chunk: Optional[int] = None, eps: float = 1e-6, *,
                    loss: Optional[torch.Tensor] = None,
                    grad_x: Optional[torch.Tensor] = None,
                    grad_gamma: Optional[torch.Tensor] = None,
                    grad_W: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """Mean cross-entropy loss of rmsnorm(x; gamma, eps) W^T against targets
    via ``flce_fwd_bwd_rmsnorm``.  Returns (loss [] fp32, grad_x like x,
    grad_gamma [H] fp32, grad_W [V, H] fp32)."""
    lib = load()
    _need_cuda(x, gamma, W, targets)
    if targets.dtype != torch.int32:
        raise TypeError("targets must be int32")
    if W.dtype != x.dtype or gamma.dtype != x.dtype:
        raise TypeError("x, gamma and W must share a dtype")
    N, H = x.shape
    V = W.shape[0]
    if gamma.shape != (H,):
        raise ValueError("gamma must have shape [H]")
    chunk = N if chunk is None else int(chunk)
    dt = _dt(x)
    dev = x.device
    if loss is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
    if grad_x is None:
        grad_x = torch.empty_like(x)
    if grad_gamma is None:
        grad_gamma = torch.empty(H, dtype=torch.float32, device=dev)
    if grad_W is None:
        grad_W = torch.empty((V, H), dtype=torch.float32, device=dev)
    need = int(lib.flce_rmsnorm_workspace_bytes(N, H, V, chunk, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need_cuda(loss, grad_x, grad_gamma, grad_W, workspace)
    st = lib.flce_fwd_bwd_rmsnorm(x.data_ptr(), gamma.data_ptr(), float(eps), W.data_ptr(),
                                  targets.data_ptr(), N, H, V, chunk, loss.data_ptr(),
                                  grad_x.data_ptr(), grad_gamma.data_ptr(), grad_W.data_ptr(),
                                  workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), dt,
                                  _stream_ptr(dev))
    _check(st)
    return loss, grad_x, grad_gamma, grad_W


def orpo_workspace_bytes(pairs: int, seq_len: int, H: int, V: int, chunk_pairs: int,
                         dtype: torch.dtype) -> int:
    """Workspace of ``flce_orpo_fwd_bwd`` (0 when the shape is unsupported)."""
    dt = FLCE_BF16 if dtype == torch.bfloat16 else FLCE_F32
    return int(load().flce_orpo_workspace_bytes(pairs, seq_len, H, V, chunk_pairs, dt))


def orpo_fwd_bwd(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, pairs: int,
                 seq_len: int, beta: float = 0.1, chunk_pairs: Optional[int] = None, *,
                 loss: Optional[torch.Tensor] = None,
                 seq_logp: Optional[torch.Tensor] = None,
                 grad_h: Optional[torch.Tensor] = None,
                 grad_W: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None,
                 ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """Odds-ratio preference loss via ``flce_orpo_fwd_bwd``: rows of h and
    targets are 2 * pairs sequences of seq_len tokens, the chosen responses
    first; a negative target marks a row that does not count.  Returns
    (loss [] fp32, seq_logp [2 pairs] fp32, grad_h like h, grad_W [V, H] fp32)."""
    lib = load()
    _need_cuda(h, W, targets)
    if targets.dtype != torch.int32:
        raise TypeError("targets must be int32")
    if W.dtype != h.dtype:
        raise TypeError("h and W must share a dtype")
    N, H = h.shape
    V = W.shape[0]
    if N != 2 * pairs * seq_len or targets.shape != (N,):
        raise ValueError("h and targets must hold 2 * pairs * seq_len rows")
    chunk_pairs = pairs if chunk_pairs is None else int(chunk_pairs)
    dt = _dt(h)
    dev = h.device
    if loss is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
    if seq_logp is None:
        seq_logp = torch.empty(2 * pairs, dtype=torch.float32, device=dev)
    if grad_h is None:
        grad_h = torch.empty_like(h)
    if grad_W is None:
        grad_W = torch.empty((V, H), dtype=torch.float32, device=dev)
    need = int(lib.flce_orpo_workspace_bytes(pairs, seq_len, H, V, chunk_pairs, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need_cuda(loss, seq_logp, grad_h, grad_W, workspace)
    st = lib.flce_orpo_fwd_bwd(h.data_ptr(), W.data_ptr(), targets.data_ptr(), pairs, seq_len,
                               H, V, chunk_pairs, float(beta), loss.data_ptr(),
                               seq_logp.data_ptr(), grad_h.data_ptr(), grad_W.data_ptr(),
                               workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), dt,
                               _stream_ptr(dev))
    _check(st)
    return loss, seq_logp, grad_h, grad_W


def logits(h: torch.Tensor, W: torch.Tensor, z: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 logits h W^T via ``flce_logits`` (the first step alone)."""
    lib = load()
    _need_cuda(h, W)
    rows, H = h.shape
    V = W.shape[0]
    if z is None:
        z = torch.empty((rows, V), dtype=torch.float32, device=h.device)
    _need_cuda(z)
    _check(lib.flce_logits(h.data_ptr(), W.data_ptr(), rows, H, V, z.data_ptr(), z.stride(0),
                           _dt(h), _stream_ptr(h.device)))
    return z


def ce_rows(z: torch.Tensor, targets: torch.Tensor, scale: float, out_dtype: torch.dtype,
            row_loss: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Row losses of fp32 logits z, rewriting z in place with the scaled
    logit gradient (``flce_ce_rows``).  For bf16 the gradient of row i is
    z.view(int16)[i, :V] viewed with a pitch of 2 * z.stride(0)."""
    lib = load()
    _need_cuda(z, targets)
    if z.dtype != torch.float32 or targets.dtype != torch.int32:
        raise TypeError("z must be float32 and targets int32")
    rows, V = z.shape
    if row_loss is None:
        row_loss = torch.empty(rows, dtype=torch.float32, device=z.device)
    dt = FLCE_BF16 if out_dtype == torch.bfloat16 else FLCE_F32
    _check(lib.flce_ce_rows(z.data_ptr(), z.stride(0), targets.data_ptr(), rows, V,
                            float(scale), row_loss.data_ptr(), 1, dt,
                            _stream_ptr(z.device)))
    return row_loss


def scale_grads(grad_h: Optional[torch.Tensor], grad_W: Optional[torch.Tensor],
                scale: torch.Tensor) -> None:
    """grad_h *= scale and grad_W *= scale in place (``flce_scale_grads``);
    ``scale`` is a one-element fp32 tensor on the GPU, read by the kernel."""
    lib = load()
    _need_cuda(scale)
    if scale.dtype != torch.float32 or scale.numel() != 1:
        raise TypeError("scale must be a one-element float32 tensor")
    dev = scale.device
    dt = FLCE_BF16
    ph, nh, pw, nw = None, 0, None, 0
    if grad_h is not None:
        _need_cuda(grad_h)
        dt = _dt(grad_h)
        ph, nh = grad_h.data_ptr(), grad_h.numel()
    if grad_W is not None:
        _need_cuda(grad_W)
        if grad_W.dtype != torch.float32:
            raise TypeError("grad_W must be float32")
        pw, nw = grad_W.data_ptr(), grad_W.numel()
    _check(lib.flce_scale_grads(ph, nh, pw, nw, scale.data_ptr(), dt, _stream_ptr(dev)))


def mfma_rate(operands: torch.Tensor, iters: int, workgroups: int
              ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Matrix-core rate microbenchmark (``flce_mfma_rate``): ``workgroups``
    x 4 waves each run ``iters`` rounds of 16 bf16 32x32x16 MFMAs on
    fragments taken from ``operands`` (a contiguous GPU tensor of at least
    8 KiB, whole 16-byte pieces).  Returns (sink [4 * workgroups] fp32: per
    wave, the sum over its lanes l and 16 blocks of the block's result at
    row 4 * (l // 32), column l % 32; clocks [4 * workgroups, 2] int64: the
    shader clocks and 100 MHz reference ticks each wave spent in its loop)."""
    lib = load()
    _need_cuda(operands)
    if not operands.is_contiguous():
        raise ValueError("operands must be contiguous")
    dev = operands.device
    nbytes = operands.numel() * operands.element_size()
    sink = torch.empty(4 * workgroups, dtype=torch.float32, device=dev)
    clocks = torch.empty((4 * workgroups, 2), dtype=torch.int64, device=dev)
    _check(lib.flce_mfma_rate(operands.data_ptr(), nbytes, int(iters), int(workgroups),
                              sink.data_ptr(), clocks.data_ptr(), _stream_ptr(dev)))
    return sink, clocks


class LinearCrossEntropyFunction(torch.autograd.Function):
    """Autograd node for the fused head: the forward call computes the mean
    loss and both gradients at once; backward only scales them by the
    incoming gradient of the loss (on the GPU, without a host sync).  The
    returned gradient of W is fp32; autograd casts it to W's dtype when it
    accumulates into W.grad.  One backward per forward (the stored
    gradients are scaled in place)."""

    @staticmethod
    def forward(ctx, h, W, targets, chunk):
        loss, grad_h, grad_W = fwd_bwd(h.detach(), W.detach(), targets, chunk)
        ctx.save_for_backward(grad_h, grad_W)
        return loss

    @staticmethod
    def backward(ctx, grad_out):
        grad_h, grad_W = ctx.saved_tensors
        need_h, need_W = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        scale = grad_out.detach().to(torch.float32).reshape(1).contiguous()
        scale_grads(grad_h if need_h else None, grad_W if need_W else None, scale)
        return (grad_h if need_h else None, grad_W if need_W else None, None, None)


def linear_cross_entropy(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                         chunk: Optional[int] = None) -> torch.Tensor:
    """Mean cross entropy of h W^T against int32 targets as a differentiable
    op (the logits are never materialised)."""
    return LinearCrossEntropyFunction.apply(h, W, targets, chunk)


def cross_entropy_(logits: torch.Tensor, targets: torch.Tensor,
                   loss: Optional[torch.Tensor] = None,
                   row_loss: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Mean cross entropy of 2-D ``logits`` (bf16 or fp32) against int32
    ``targets`` via ``flce_cross_entropy``; ``logits`` is overwritten with
    dloss/dlogits (the trailing underscore: in place).  Returns the loss."""
    lib = load()
    _need_cuda(targets)
    if not logits.is_cuda or logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be a 2-D GPU tensor with unit column stride")
    if targets.dtype != torch.int32:
        raise TypeError("targets must be int32")
    rows, V = logits.shape
    dev = logits.device
    if loss is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
    if row_loss is None:
        row_loss = torch.empty(rows, dtype=torch.float32, device=dev)
    _need_cuda(loss, row_loss)
    _check(lib.flce_cross_entropy(logits.data_ptr(), logits.stride(0), targets.data_ptr(), rows,
                                  V, loss.data_ptr(), row_loss.data_ptr(), _dt(logits),
                                  _stream_ptr(dev)))
    return loss


class CrossEntropyFunction(torch.autograd.Function):
    """Autograd node for the cross entropy on given logits: the forward call
    computes the mean loss and turns the logits' own memory into their
    gradient (the logits tensor is consumed); backward scales it by the
    incoming gradient of the loss.  One backward per forward."""

    @staticmethod
    def forward(ctx, logits, targets):
        buf = logits.detach()
        loss = cross_entropy_(buf, targets)
        ctx.save_for_backward(buf)
        return loss

    @staticmethod
    def backward(ctx, grad_out):
        (g,) = ctx.saved_tensors
        scale = grad_out.detach().to(torch.float32).reshape(1).contiguous()
        if g.dtype == torch.float32:
            scale_grads(None, g.view(-1), scale)
        else:
            scale_grads(g.view(-1), None, scale)
        return g, None


def cross_entropy(logits: torch.Tensor, targets: torch.Tensor) -> torch.Tensor:
    """Differentiable mean cross entropy on given logits; the logits' memory
    holds their gradient afterwards (do not reuse the logits)."""
    return CrossEntropyFunction.apply(logits, targets)
