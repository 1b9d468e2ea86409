"""ctypes marshalling for libgrpo.so.  No arithmetic of the loss happens here."""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_DTYPE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p


class GRPOError(RuntimeError):
    """A negative grpo_status returned by the library."""


class GRPOOptions(ctypes.Structure):
    """Mirror of struct grpo_options."""
    _fields_ = [("kl_estimator", ctypes.c_int), ("detach_ratio", ctypes.c_int),
                ("normalization", ctypes.c_int), ("temperature", ctypes.c_float),
                ("fp8_logits", ctypes.c_int), ("chunk_rows", ctypes.c_int),
                ("vocab_piece", ctypes.c_int),
                ("trace_kernel", ctypes.c_int), ("trace_capacity", ctypes.c_int),
                ("trace_events", ctypes.POINTER(ctypes.c_void_p)),
                ("trace_count", ctypes.POINTER(ctypes.c_int)),
                ("dx_host", ctypes.c_void_p), ("dw_host", ctypes.c_void_p),
                ("copy_stream", ctypes.c_void_p)]


TRACE_KERNELS = {"none": 0, "fwd_all": 1, "fwd_chunk": 2, "recompute": 3, "dx": 4, "dw": 5}


class KernelTrace:
    """Event pairs for grpo_options' kernel tracing: the library records them on the call's
    stream around each launch of one kernel.  ``events`` are torch.cuda.Event objects with
    timing enabled, already recorded once (so that their HIP events exist)."""

    def __init__(self, kernel: str, events):
        self.kernel = TRACE_KERNELS[kernel]
        self.events = list(events)
        self._handles = (ctypes.c_void_p * len(self.events))(*[e.cuda_event for e in self.events])
        self.count = ctypes.c_int(0)

    def attach(self, o: "GRPOOptions") -> "GRPOOptions":
        o.trace_kernel = self.kernel
        o.trace_capacity = len(self.events) // 2
        o.trace_events = ctypes.cast(self._handles, ctypes.POINTER(ctypes.c_void_p))
        o.trace_count = ctypes.pointer(self.count)
        return o

    def launch_ms(self):
        """Milliseconds of each bracketed launch of the last call (after a synchronise)."""
        n = min(self.count.value, len(self.events) // 2)
        return [self.events[2 * i].elapsed_time(self.events[2 * i + 1]) for i in range(n)]


KL_ESTIMATORS = {"reverse": 0, "forward": 1, "reverse_q": 2}
NORMALIZATIONS = {"tokens": 0, "sequences": 1}


def options(kl: str = "reverse", detach: bool = True, norm: str = "tokens",
            temperature: float = 1.0, fp8_logits: bool = False,
            chunk_rows: int = 0, vocab_piece: int = 0) -> GRPOOptions:
    """A grpo_options value from names (the library validates the ranges).  chunk_rows:
    loss rows per backward chunk; vocab_piece: vocabulary entries per piece of a chunk's
    softmax terms (0: the library's defaults)."""
    return GRPOOptions(KL_ESTIMATORS[kl], int(bool(detach)), NORMALIZATIONS[norm],
                       float(temperature), int(bool(fp8_logits)), int(chunk_rows),
                       int(vocab_piece))


def _as_options(o):
    if o is None or isinstance(o, GRPOOptions):
        return o
    return options(**o)


def _opts(o):
    o = _as_options(o)
    return None if o is None else ctypes.byref(o)


def _copy_options(o) -> GRPOOptions:
    """A separate GRPOOptions holding o's fields (the library's defaults for None)."""
    o = _as_options(o)
    c = GRPOOptions()
    if o is None:
        _LIB.grpo_default_options(ctypes.byref(c))
    else:
        ctypes.memmove(ctypes.byref(c), ctypes.byref(o), ctypes.sizeof(c))
    return c


_COPY_STREAMS = {}


def offload_stream(device=None) -> torch.cuda.Stream:
    """The stream the gradient offload copies on, one per device, created with the
    default priority (as every stream here is)."""
    dev = torch.device("cuda", torch.cuda.current_device() if device is None
                       else torch.device(device).index or 0)
    s = _COPY_STREAMS.get(dev.index)
    if s is None:
        s = _COPY_STREAMS[dev.index] = torch.cuda.Stream(device=dev)
    return s


def _need_host(t: torch.Tensor, name: str, dtype, shape):
    if t.is_cuda or not t.is_pinned():
        raise ValueError(f"{name} must be pinned host memory (pin_memory=True)")
    if not t.is_contiguous() or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


def library_path() -> str:
    return os.path.join(_HERE, "libgrpo.so")


def load_library():
    """Load libgrpo.so (once) and declare the exported signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python grpo_loss_amd/build.py` first")
    lib = ctypes.CDLL(path)
    lib.grpo_status_string.restype = ctypes.c_char_p
    lib.grpo_status_string.argtypes = [ctypes.c_int]
    lib.grpo_workspace_bytes.restype = ctypes.c_size_t
    lib.grpo_workspace_bytes.argtypes = [_c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_int, ctypes.c_int]
    lib.grpo_workspace_bytes_opts.restype = ctypes.c_size_t
    lib.grpo_workspace_bytes_opts.argtypes = [_c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_int,
                                              ctypes.c_int, ctypes.POINTER(GRPOOptions)]
    lib.grpo_quantize_e4m3.restype = ctypes.c_int
    lib.grpo_quantize_e4m3.argtypes = [_c_p, ctypes.c_int, _c_i64, _c_i64, _c_p, _c_p, _c_p]
    lib.grpo_advantages.restype = ctypes.c_int
    lib.grpo_advantages.argtypes = [_c_p, _c_i64, _c_i64, _c_i64, ctypes.c_float, ctypes.c_int,
                                    _c_p, _c_p]
    lib.grpo_loss_fwd.restype = ctypes.c_int
    opt_p = ctypes.POINTER(GRPOOptions)
    lib.grpo_default_options.restype = None
    lib.grpo_default_options.argtypes = [opt_p]
    lib.grpo_loss_fwd.argtypes = [_c_p, _c_p, _c_p, ctypes.c_int, _c_p, _c_p, _c_p, _c_i64,
                                  _c_i64, _c_i64, _c_i64, ctypes.c_float, _c_p, _c_p, _c_p, _c_p,
                                  _c_p, _c_p, opt_p, _c_p, ctypes.c_size_t, _c_p]
    lib.grpo_loss_fwd_noalloc.restype = ctypes.c_int
    lib.grpo_loss_fwd_noalloc.argtypes = [_c_p, _c_p, _c_p, ctypes.c_int, _c_p, _c_p, _c_p,
                                          _c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_float, _c_p,
                                          _c_p, _c_p, _c_p, _c_p, _c_p, opt_p, _c_p]
    lib.grpo_loss_bwd.restype = ctypes.c_int
    lib.grpo_loss_bwd.argtypes = [_c_p, _c_p, ctypes.c_int, _c_p, _c_p, _c_p, _c_i64, _c_i64,
                                  _c_i64, _c_i64, _c_p, ctypes.c_float, _c_p, _c_p, ctypes.c_int,
                                  _c_p, opt_p, _c_p, ctypes.c_size_t, _c_p]
    lib.grpo_loss_fwd_bwd.restype = ctypes.c_int
    lib.grpo_loss_fwd_bwd.argtypes = [_c_p, _c_p, _c_p, ctypes.c_int, _c_p, _c_p, _c_p, _c_i64,
                                      _c_i64, _c_i64, _c_i64, ctypes.c_float, _c_p,
                                      ctypes.c_float, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                      _c_p, ctypes.c_int, _c_p, opt_p, _c_p, ctypes.c_size_t,
                                      _c_p]
    lib.grpo_scale_grad.restype = ctypes.c_int
    lib.grpo_scale_grad.argtypes = [_c_p, ctypes.c_int, _c_i64, _c_i64, _c_p, _c_i64, _c_p,
                                    ctypes.c_float, _c_p, _c_p]
    lib.grpo_restore_workspace_bytes.restype = ctypes.c_size_t
    lib.grpo_restore_workspace_bytes.argtypes = [_c_i64, _c_i64]
    lib.grpo_grad_restore.restype = ctypes.c_int
    lib.grpo_grad_restore.argtypes = [_c_p, _c_p, ctypes.c_int, _c_p, _c_i64, _c_i64, _c_i64,
                                      _c_i64, _c_p, ctypes.c_float, _c_p, _c_p, _c_p, _c_p,
                                      ctypes.c_size_t, _c_p]
    _LIB = lib
    return lib


load_library()


def _check(rc: int):
    if rc != 0:
        msg = _LIB.grpo_status_string(rc).decode()
        raise GRPOError(f"libgrpo returned {rc}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPE[t.dtype]


def _need(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def grpo_workspace_bytes(S: int, L: int, H: int, V: int, dtype: torch.dtype,
                         need_dW: bool = False, opts=None) -> int:
    if opts is None:
        return int(_LIB.grpo_workspace_bytes(S, L, H, V, _DTYPE[dtype], int(bool(need_dW))))
    return int(_LIB.grpo_workspace_bytes_opts(S, L, H, V, _DTYPE[dtype], int(bool(need_dW)),
                                              _opts(opts)))


def grpo_quantize_e4m3(x: torch.Tensor, stream=None):
    """Per-row e4m3 quantisation of a [rows, H] device matrix: (codes uint8 [rows, H],
    scales float32 [rows])."""
    _need(x, "x")
    rows, H = x.shape
    codes = torch.empty(rows, H, dtype=torch.uint8, device=x.device)
    scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(_LIB.grpo_quantize_e4m3(_ptr(x), _dt(x), rows, H, _ptr(codes), _ptr(scales),
                                   _stream(stream)))
    return codes, scales


def grpo_advantages(rewards: torch.Tensor, eps: float = 1e-4, unbiased: bool = True,
                    out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """rewards fp32 [B, G] or [B, G, K] on the device -> advantages fp32 [B*G]."""
    _need(rewards, "rewards")
    if rewards.dtype != torch.float32:
        raise TypeError("rewards must be float32")
    r = rewards if rewards.dim() == 3 else rewards.unsqueeze(-1)
    B, G, K = r.shape
    if out is None:
        out = torch.empty(B * G, dtype=torch.float32, device=rewards.device)
    _check(_LIB.grpo_advantages(_ptr(r), B, G, K, eps, int(bool(unbiased)), _ptr(out),
                                _stream(stream)))
    return out


def _shape(xq: torch.Tensor, L: int | None):
    if xq.dim() == 3:
        S, L2, H = xq.shape
        if L is not None and L != L2:
            raise ValueError("L does not match X's shape")
        return S, L2, H
    if xq.dim() != 2 or L is None or xq.shape[0] % L:
        raise ValueError("X must be [S, L, H], or [S*L, H] with L given")
    return xq.shape[0] // L, L, xq.shape[1]


def grpo_loss_fwd(xq, xp, W, targets, mask, adv, beta: float = 0.04, L: int | None = None,
                  workspace: torch.Tensor | None = None, want_terms: bool = True, stream=None,
                  opts=None):
    """Forward.  Returns dict(loss [1], saved [N, 4], logp, ref_logp, kl [N] (or None),
    status int32 [1], workspace).  opts: a GRPOOptions, a dict of options(...) keywords,
    or None for the defaults."""
    for t, n in ((xq, "xq"), (xp, "xp"), (W, "W"), (targets, "targets"), (mask, "mask"),
                 (adv, "adv")):
        _need(t, n)
    S, L, H = _shape(xq, L)
    V = W.shape[0]
    dt = _dt(xq)
    if xp.dtype != xq.dtype or W.dtype != xq.dtype:
        raise TypeError("xq, xp and W must share one dtype")
    if targets.dtype != torch.int64 or mask.dtype != torch.uint8 or adv.dtype != torch.float32:
        raise TypeError("targets int64, mask uint8, adv float32 expected")
    dev = xq.device
    N = S * L
    need = grpo_workspace_bytes(S, L, H, V, xq.dtype, False, opts)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    loss = torch.empty(1, **f32)
    saved = torch.empty(N, 4, **f32)
    terms = [torch.empty(N, **f32) for _ in range(3)] if want_terms else [None] * 3
    status = torch.empty(1, dtype=torch.int32, device=dev)
    _check(_LIB.grpo_loss_fwd(_ptr(xq), _ptr(xp), _ptr(W), dt, _ptr(targets), _ptr(mask),
                              _ptr(adv), S, L, H, V, beta, _ptr(loss), _ptr(saved),
                              _ptr(terms[0]), _ptr(terms[1]), _ptr(terms[2]), _ptr(status),
                              _opts(opts), _ptr(workspace), workspace.numel(), _stream(stream)))
    return {"loss": loss, "saved": saved, "logp": terms[0], "ref_logp": terms[1],
            "kl": terms[2], "status": status, "workspace": workspace}


def grpo_loss_fwd_noalloc(xq, xp, W, targets, mask, adv, beta: float = 0.04,
                          L: int | None = None, want_terms: bool = True, stream=None,
                          opts=None):
    """grpo_loss_fwd without a workspace: the library uses its fixed per-GPU scratch
    array (GRPOError with GRPO_ERR_SCRATCH when the sizes need more).  Returns dict(loss,
    saved, logp, ref_logp, kl, status); the outputs are allocated here, by the caller."""
    for t, n in ((xq, "xq"), (xp, "xp"), (W, "W"), (targets, "targets"), (mask, "mask"),
                 (adv, "adv")):
        _need(t, n)
    S, L, H = _shape(xq, L)
    V = W.shape[0]
    dt = _dt(xq)
    if xp.dtype != xq.dtype or W.dtype != xq.dtype:
        raise TypeError("xq, xp and W must share one dtype")
    if targets.dtype != torch.int64 or mask.dtype != torch.uint8 or adv.dtype != torch.float32:
        raise TypeError("targets int64, mask uint8, adv float32 expected")
    dev = xq.device
    N = S * L
    f32 = dict(dtype=torch.float32, device=dev)
    loss = torch.empty(1, **f32)
    saved = torch.empty(N, 4, **f32)
    terms = [torch.empty(N, **f32) for _ in range(3)] if want_terms else [None] * 3
    status = torch.empty(1, dtype=torch.int32, device=dev)
    _check(_LIB.grpo_loss_fwd_noalloc(_ptr(xq), _ptr(xp), _ptr(W), dt, _ptr(targets),
                                      _ptr(mask), _ptr(adv), S, L, H, V, beta, _ptr(loss),
                                      _ptr(saved), _ptr(terms[0]), _ptr(terms[1]),
                                      _ptr(terms[2]), _ptr(status), _opts(opts),
                                      _stream(stream)))
    return {"loss": loss, "saved": saved, "logp": terms[0], "ref_logp": terms[1],
            "kl": terms[2], "status": status}


def grpo_loss_bwd(xq, W, targets, mask, saved, L: int | None = None, grad_loss=None,
                  loss_scale: float = 1.0, need_dW: bool = False, dW: torch.Tensor | None = None,
                  accumulate_dW: bool = False, found_inf: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, dXq: torch.Tensor | None = None,
                  stream=None, opts=None):
    """Backward.  Returns dict(dXq, dW (or None), found_inf, workspace).  opts: the
    options given to the forward."""
    for t, n in ((xq, "xq"), (W, "W"), (targets, "targets"), (mask, "mask"), (saved, "saved")):
        _need(t, n)
    S, L, H = _shape(xq, L)
    V = W.shape[0]
    dev = xq.device
    need_dW = need_dW or dW is not None
    need = grpo_workspace_bytes(S, L, H, V, xq.dtype, need_dW, opts)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if dXq is None:
        dXq = torch.empty_like(xq)
    if need_dW and dW is None:
        dW = torch.empty(V, H, dtype=torch.float32, device=dev)
    if found_inf is None:
        found_inf = torch.zeros(1, dtype=torch.int32, device=dev)
    if grad_loss is not None:
        _need(grad_loss, "grad_loss")
    _check(_LIB.grpo_loss_bwd(_ptr(xq), _ptr(W), _dt(xq), _ptr(targets), _ptr(mask),
                              _ptr(saved), S, L, H, V, _ptr(grad_loss), float(loss_scale),
                              _ptr(dXq), _ptr(dW) if need_dW else None, int(bool(accumulate_dW)),
                              _ptr(found_inf), _opts(opts), _ptr(workspace), workspace.numel(),
                              _stream(stream)))
    return {"dXq": dXq, "dW": dW if need_dW else None, "found_inf": found_inf,
            "workspace": workspace}


def grpo_loss_fwd_bwd(xq, xp, W, targets, mask, adv, beta: float = 0.04, L: int | None = None,
                      grad_loss=None, loss_scale: float = 1.0, need_dW: bool = False,
                      dW: torch.Tensor | None = None, accumulate_dW: bool = False,
                      found_inf: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, dXq: torch.Tensor | None = None,
                      want_terms: bool = True, stream=None, opts=None,
                      dx_host: torch.Tensor | None = None, dw_host: torch.Tensor | None = None,
                      copy_stream=None):
    """Forward and backward in one call (the policy logits are computed once).  Returns
    dict(loss, saved, logp, ref_logp, kl, status, dXq, dW (or None), found_inf,
    workspace).

    Gradient offload: dx_host (pinned host [S*L, H] in X's dtype) receives dX in loss-row
    order instead of a device dXq (returned as None), dw_host (pinned host [V, H] fp32)
    receives dW; both are copied on copy_stream (default: offload_stream()) while later
    chunks compute.  grpo_grad_restore brings them back."""
    for t, n in ((xq, "xq"), (xp, "xp"), (W, "W"), (targets, "targets"), (mask, "mask"),
                 (adv, "adv")):
        _need(t, n)
    S, L, H = _shape(xq, L)
    V = W.shape[0]
    dt = _dt(xq)
    if xp.dtype != xq.dtype or W.dtype != xq.dtype:
        raise TypeError("xq, xp and W must share one dtype")
    if targets.dtype != torch.int64 or mask.dtype != torch.uint8 or adv.dtype != torch.float32:
        raise TypeError("targets int64, mask uint8, adv float32 expected")
    dev = xq.device
    N = S * L
    need_dW = need_dW or dW is not None or dw_host is not None
    if dx_host is not None or dw_host is not None:
        opts = _copy_options(opts)
        cs = offload_stream(dev) if copy_stream is None else copy_stream
        opts.copy_stream = cs.cuda_stream
        if dx_host is not None:
            if dXq is not None:
                raise ValueError("dXq and dx_host are exclusive")
            _need_host(dx_host, "dx_host", xq.dtype, (N, H))
            opts.dx_host = dx_host.data_ptr()
        if dw_host is not None:
            _need_host(dw_host, "dw_host", torch.float32, (V, H))
            opts.dw_host = dw_host.data_ptr()
    need = grpo_workspace_bytes(S, L, H, V, xq.dtype, need_dW, opts)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    loss = torch.empty(1, **f32)
    saved = torch.empty(N, 4, **f32)
    terms = [torch.empty(N, **f32) for _ in range(3)] if want_terms else [None] * 3
    status = torch.empty(1, dtype=torch.int32, device=dev)
    if dXq is None and dx_host is None:
        dXq = torch.empty_like(xq)
    if need_dW and dW is None:
        dW = torch.empty(V, H, **f32)
    if found_inf is None:
        found_inf = torch.zeros(1, dtype=torch.int32, device=dev)
    if grad_loss is not None:
        _need(grad_loss, "grad_loss")
    _check(_LIB.grpo_loss_fwd_bwd(_ptr(xq), _ptr(xp), _ptr(W), dt, _ptr(targets), _ptr(mask),
                                  _ptr(adv), S, L, H, V, beta, _ptr(grad_loss),
                                  float(loss_scale), _ptr(loss), _ptr(saved), _ptr(terms[0]),
                                  _ptr(terms[1]), _ptr(terms[2]), _ptr(status), _ptr(dXq),
                                  _ptr(dW) if need_dW else None, int(bool(accumulate_dW)),
                                  _ptr(found_inf), _opts(opts), _ptr(workspace),
                                  workspace.numel(), _stream(stream)))
    return {"loss": loss, "saved": saved, "logp": terms[0], "ref_logp": terms[1],
            "kl": terms[2], "status": status, "dXq": dXq, "dW": dW if need_dW else None,
            "found_inf": found_inf, "workspace": workspace}


def grpo_restore_workspace_bytes(N: int) -> int:
    return int(_LIB.grpo_restore_workspace_bytes(1, N))


def grpo_grad_restore(mask, dx_host=None, dw_host=None, grad_loss=None, loss_scale: float = 1.0,
                      dXq=None, dW=None, found_inf=None, workspace=None, stream=None):
    """The way back of the gradient offload: dXq [S*L, H] (device, X's dtype; masked rows
    0) from dx_host, and dW [V, H] fp32 from dw_host, both times grad_loss / loss_scale as
    grpo_scale_grad applies it; the kernels read the pinned host tensors directly.
    Returns dict(dXq, dW, found_inf).  The host tensors must stay alive until the kernels
    enqueued on `stream` have run."""
    if dx_host is None and dw_host is None:
        raise ValueError("nothing to restore")
    _need(mask, "mask")
    N = mask.numel()
    dev = mask.device
    H = (dx_host if dx_host is not None else dw_host).shape[1]
    V = dw_host.shape[0] if dw_host is not None else 0
    if dx_host is not None:
        _need_host(dx_host, "dx_host", dx_host.dtype, (N, H))
        if dXq is None:
            dXq = torch.empty(N, H, dtype=dx_host.dtype, device=dev)
        _need(dXq, "dXq")
    if dw_host is not None:
        _need_host(dw_host, "dw_host", torch.float32, (V, H))
        if dW is None:
            dW = torch.empty(V, H, dtype=torch.float32, device=dev)
        _need(dW, "dW")
    dtype = (dx_host if dx_host is not None else dw_host).dtype
    if found_inf is None:
        found_inf = torch.zeros(1, dtype=torch.int32, device=dev)
    if grad_loss is not None:
        _need(grad_loss, "grad_loss")
    need = grpo_restore_workspace_bytes(N)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(_LIB.grpo_grad_restore(_ptr(dx_host), _ptr(dw_host), _DTYPE[dtype], _ptr(mask), 1, N,
                                  H, V, _ptr(grad_loss), float(loss_scale),
                                  _ptr(dXq) if dx_host is not None else None,
                                  _ptr(dW) if dw_host is not None else None, _ptr(found_inf),
                                  _ptr(workspace), workspace.numel(), _stream(stream)))
    return {"dXq": dXq if dx_host is not None else None,
            "dW": dW if dw_host is not None else None, "found_inf": found_inf}


class _PinnedPool:
    """Pinned host buffers of the autograd offload, reused across steps.  A buffer is out
    from the forward that fills it until its restore is enqueued; the copies that touch it
    all run on the device's one offload stream, in order, so a later forward's copies into
    a returned buffer follow the restore's copies out of it."""

    def __init__(self):
        self._free = {}

    def take(self, shape, dtype, device):
        key = (tuple(shape), dtype, torch.device(device).index)
        lst = self._free.get(key)
        if lst:
            return lst.pop()
        return torch.empty(shape, dtype=dtype, pin_memory=True)

    def give(self, t, device):
        if t is not None:
            self._free.setdefault((tuple(t.shape), t.dtype, torch.device(device).index),
                                  []).append(t)


_PINNED = _PinnedPool()


def grpo_scale_grad(dXq, grad_loss, loss_scale: float = 1.0, dW=None, found_inf=None,
                    stream=None):
    """dXq (and dW) *= grad_loss / loss_scale in place; returns found_inf."""
    _need(dXq, "dXq")
    _need(grad_loss, "grad_loss")
    H = dXq.shape[-1]
    rows = dXq.numel() // H
    if found_inf is None:
        found_inf = torch.zeros(1, dtype=torch.int32, device=dXq.device)
    V = 0
    if dW is not None:
        _need(dW, "dW")
        if dW.dtype != torch.float32 or dW.shape[-1] != H:
            raise TypeError("dW must be float32 [V, H]")
        V = dW.shape[0]
    _check(_LIB.grpo_scale_grad(_ptr(dXq), _dt(dXq), rows, H, _ptr(dW), V, _ptr(grad_loss),
                                float(loss_scale), _ptr(found_inf), _stream(stream)))
    return found_inf


class _GRPOLoss(torch.autograd.Function):
    @staticmethod
    def forward(ctx, xq, xp, W, targets, mask, adv, beta, L, loss_scale, need_dW, opts,
                single_pass, offload, grad_hint):
        ctx.L, ctx.loss_scale, ctx.need_dW, ctx.opts = L, loss_scale, need_dW, opts
        ctx.single_pass, ctx.offload = single_pass, offload
        ctx.w_dtype = W.dtype
        if single_pass:
            # the gradients now, for an upstream gradient of grad_hint: they are narrowed to
            # X's dtype with it applied, and the backward multiplies them by
            # grad / grad_hint, exactly 1 when the hint was right
            ctx.hint = float(loss_scale if grad_hint is None else grad_hint)
            want_dW = need_dW and ctx.needs_input_grad[2]
            dev = xq.device
            host = {}
            if offload:
                N, H = targets.numel(), xq.shape[-1]
                host["dx_host"] = _PINNED.take((N, H), xq.dtype, dev)
                if want_dW:
                    host["dw_host"] = _PINNED.take((W.shape[0], H), torch.float32, dev)
            hint = torch.full((1,), ctx.hint, dtype=torch.float32, device=dev)
            out = grpo_loss_fwd_bwd(xq, xp, W, targets, mask, adv, beta, L, hint, loss_scale,
                                    need_dW=want_dW, want_terms=False, opts=opts, **host)
            if offload:
                # device dX was never written and device dW is dropped here: both live in
                # host memory until the backward
                ctx.host = (host.get("dx_host"), host.get("dw_host"), mask, dev, xq.shape)
                ctx.grads = (None, None, out["found_inf"])
            else:
                ctx.grads = (out["dXq"], out["dW"], out["found_inf"])
            ctx.mark_non_differentiable(out["status"])
            return out["loss"][0], out["status"]
        out = grpo_loss_fwd(xq, xp, W, targets, mask, adv, beta, L, want_terms=False,
                            opts=opts)
        ctx.save_for_backward(xq, W, targets, mask, out["saved"])
        ctx.workspace = out["workspace"]
        ctx.mark_non_differentiable(out["status"])
        return out["loss"][0], out["status"]

    @staticmethod
    def backward(ctx, grad_loss, _grad_status):
        g = grad_loss.reshape(1).to(torch.float32).contiguous()
        nones = (None,) * 11  # targets .. grad_hint
        if ctx.single_pass:
            dX, dW32, found = ctx.grads
            ctx.grads = None
            if ctx.offload:
                dx_host, dw_host, mask, dev, xshape = ctx.host
                ctx.host = None
                r = grpo_grad_restore(mask, dx_host, dw_host, g, ctx.hint, found_inf=found)
                dX, dW32 = r["dXq"].view(xshape), r["dW"]
                _PINNED.give(dx_host, dev)
                _PINNED.give(dw_host, dev)
            else:
                grpo_scale_grad(dX, g, ctx.hint, dW=dW32, found_inf=found)
            ctx.found_inf = found
            dW = dW32.to(ctx.w_dtype) if dW32 is not None else None
            return (dX, None, dW) + nones
        xq, W, targets, mask, saved = ctx.saved_tensors
        out = grpo_loss_bwd(xq, W, targets, mask, saved, ctx.L, g, ctx.loss_scale,
                            need_dW=ctx.need_dW and W.requires_grad, workspace=None,
                            opts=ctx.opts)
        dW = out["dW"].to(W.dtype) if out["dW"] is not None else None
        ctx.found_inf = out["found_inf"]
        return (out["dXq"], None, dW) + nones


def grpo_loss(xq, xp, W, targets, mask, rewards, beta: float = 0.04, eps: float = 1e-4,
              loss_scale: float = 1.0, need_dW: bool = False, L: int | None = None,
              opts=None, single_pass: bool = False, offload: bool = False,
              grad_hint: float | None = None):
    """The GRPO loss with autograd.  xq, xp [S, L, H] (or [S*L, H] with L), W [V, H],
    targets int64 and mask (bool/uint8) of S*L elements, rewards fp32 [S] or [B, G(, K)].

    Returns (loss, status).  Gradients flow to xq (and W when need_dW); xp and the
    reference path get none.  With loss scaling, back-propagate loss * loss_scale and pass
    the same loss_scale here: the returned gradients are unscaled.  opts selects the loss
    variant (see options()).

    single_pass computes the gradients during the forward (grpo_loss_fwd_bwd) and keeps
    them, X_q-sized (plus dW), until the backward.  They are narrowed to X's dtype with
    the upstream gradient grad_hint already applied (default: loss_scale, the gradient of
    loss * loss_scale); the backward multiplies them by the actual upstream gradient over
    grad_hint, which is exactly 1, and changes nothing, when the hint was right.  offload
    (single pass only) keeps them in pinned host memory instead, copied there on a second
    stream while later chunks compute and brought back by the backward
    (grpo_grad_restore); the gradients are the same bits."""
    if offload and not single_pass:
        raise ValueError("offload applies to the single pass")
    r = rewards.float()
    if r.dim() == 1:
        r = r.unsqueeze(0)
    adv = grpo_advantages(r.contiguous(), eps)
    m = mask.reshape(-1).to(torch.uint8).contiguous()
    y = targets.reshape(-1).contiguous()
    return _GRPOLoss.apply(xq.contiguous(), xp.contiguous(), W.contiguous(), y, m, adv,
                           float(beta), L if xq.dim() == 2 else xq.shape[1], float(loss_scale),
                           bool(need_dW), opts, bool(single_pass), bool(offload), grad_hint)
