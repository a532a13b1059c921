"""ctypes binding of libdspark (argument marshalling only).

Every function passes device pointers of torch tensors and torch's current
HIP stream to the C ABI declared in include/dspark.h; no step of the path is
computed here.  If the library has not been built the first call raises
RuntimeError: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_NAME = "libdspark.so"
_HERE = os.path.dirname(os.path.abspath(__file__))

DSPARK_OK, DSPARK_ERR_INVALID_ARG, DSPARK_ERR_UNSUPPORTED, DSPARK_ERR_WORKSPACE, DSPARK_ERR_HIP = range(5)
DSPARK_F32, DSPARK_BF16 = 0, 1
DSPARK_GREEDY, DSPARK_GUMBEL = 0, 1

_lib = None
_lock = threading.Lock()


class DSparkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"dspark status {status}: {message}")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


def _declare(lib):
    c_int, c_size, c_vp, c_f, c_u64 = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float, ctypes.c_uint64
    lib.dspark_draft_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int]
    lib.dspark_draft_workspace_bytes.restype = c_size
    lib.dspark_markov_draft.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int,
                                        c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_f, c_vp, c_int, c_u64,
                                        c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]
    lib.dspark_markov_draft.restype = c_int
    lib.dspark_markov_draft_noalloc.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int,
                                                c_vp, c_vp, c_vp, c_vp, c_vp,
                                                c_vp, c_f, c_vp, c_int, c_u64,
                                                c_vp, c_vp, c_vp, c_vp, c_vp]
    lib.dspark_markov_draft_noalloc.restype = c_int
    lib.dspark_rnn_draft_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int]
    lib.dspark_rnn_draft_workspace_bytes.restype = c_size
    lib.dspark_rnn_draft.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int,
                                     c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                     c_vp, c_f, c_vp, c_int, c_u64,
                                     c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]
    lib.dspark_rnn_draft.restype = c_int
    lib.dspark_gumbel_from_words.argtypes = [c_int, c_vp, c_vp, c_vp]
    lib.dspark_gumbel_from_words.restype = c_int
    lib.dspark_schedule.argtypes = [c_int, c_int, c_vp, c_vp, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]
    lib.dspark_schedule.restype = c_int
    lib.dspark_schedule_workspace_bytes.argtypes = [c_int, c_int]
    lib.dspark_schedule_workspace_bytes.restype = c_size
    lib.dspark_serve_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int]
    lib.dspark_serve_workspace_bytes.restype = c_size
    lib.dspark_step_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int]
    lib.dspark_step_workspace_bytes.restype = c_size
    lib.dspark_step.argtypes = ([c_int] * 6 + [c_vp] * 6 + [c_f, c_vp, c_int, c_u64] + [c_vp, c_vp, c_int, c_int] +
                                [c_vp] * 8 + [c_vp, c_size, c_vp])
    lib.dspark_step.restype = c_int
    lib.dspark_parallel_draft.argtypes = [c_int, c_int, c_int, c_int, c_vp, c_int, c_u64, c_vp, c_vp, c_vp]
    lib.dspark_parallel_draft.restype = c_int
    lib.dspark_set_draft_launch.argtypes = [c_int]
    lib.dspark_set_draft_launch.restype = c_int
    lib.dspark_get_draft_launch.argtypes = []
    lib.dspark_get_draft_launch.restype = c_int
    lib.dspark_schedule_threshold.argtypes = [c_int, c_int, c_vp, ctypes.c_float, c_vp, c_vp, c_vp]
    lib.dspark_schedule_threshold.restype = c_int
    lib.dspark_serve.argtypes = ([c_int] * 6 + [c_int] + [c_vp] * 6 + [ctypes.c_float, c_vp, c_int, c_u64] +
                                 [c_vp, c_vp, c_int, c_int, c_int, ctypes.c_float] + [c_vp] * 9 + [c_size, c_vp])
    lib.dspark_serve.restype = c_int
    lib.dspark_sts_workspace_bytes.argtypes = [c_int, c_int, c_int]
    lib.dspark_sts_workspace_bytes.restype = c_size
    lib.dspark_sts_fit.argtypes = [c_int, c_int, c_vp, c_vp, c_vp, c_int, c_int, c_vp, c_vp, c_vp, c_vp,
                                   c_size, c_vp]
    lib.dspark_sts_fit.restype = c_int
    lib.dspark_verify.argtypes = [c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]
    lib.dspark_verify.restype = c_int
    lib.dspark_status_string.argtypes = [c_int]
    lib.dspark_status_string.restype = ctypes.c_char_p
    lib.dspark_last_error.argtypes = []
    lib.dspark_last_error.restype = ctypes.c_char_p
    return lib


def load(path: str | None = None):
    """Load (once) and return the ctypes handle of libdspark."""
    global _lib
    with _lock:
        if _lib is None:
            p = path or library_path()
            if not os.path.exists(p):
                raise RuntimeError(f"{p} is not built: run __graft_entry__.build() first "
                                   "(the HIP library is required; there is no fallback)")
            _lib = _declare(ctypes.CDLL(p))
        return _lib


def _check(status: int):
    if status != DSPARK_OK:
        lib = load()
        msg = lib.dspark_last_error().decode() or lib.dspark_status_string(status).decode()
        raise DSparkError(status, msg)


# ----------------------------------------------------------------------------
# torch-facing wrappers
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


_ws_cache = {}


def workspace_bytes(B: int, gamma: int, V: int, r: int) -> int:
    return int(load().dspark_draft_workspace_bytes(B, gamma, V, r))


def _workspace_key(kind: str, device_index: int, stream_handle: int):
    """Cache key of a library-owned workspace: one per (kind, device, HIP
    stream).  Calls enqueued on one stream run one after another, so they
    may share a workspace; calls on different streams may overlap and must
    not (their grid-barrier counters and arg-max slots would mix)."""
    return (kind, int(device_index), int(stream_handle))


def _workspace(nbytes: int, device, kind: str = "draft", layout=None):
    """The cached workspace for the current stream of `device`, at least
    `nbytes` long.  A new one is zero-filled on that same stream, so the fill
    is ordered before the call that uses it.  A call leaves the parts that
    must start at zero (counters, arg-max slots) zero again, but where they
    sit depends on the shape: when `layout` (the shape that fixes them)
    differs from the previous call's, the reused buffer is zero-filled again
    on the stream first."""
    torch = _torch()
    index = device.index if device.index is not None else torch.cuda.current_device()
    stream = torch.cuda.current_stream(index)
    key = _workspace_key(kind, index, stream.cuda_stream)
    with _lock:
        ws, last = _ws_cache.get(key, (None, None))
        if ws is None or ws.numel() < nbytes:
            with torch.cuda.stream(stream):
                ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        elif layout != last:
            with torch.cuda.stream(stream):
                ws.zero_()
        _ws_cache[key] = (ws, layout)
    return ws


def markov_draft(anchor, U, h, W1, W2, conf_w, conf_b: float, sts_T, mode: str = "greedy",
                 seed: int = 0, out=None, workspace=None):
    """Draft gamma tokens per request with the Markov head; returns
    (tokens int32, logit fp32, conf fp32, surv fp32), each [B, gamma].

    U [B, gamma, V], h [B, gamma, d], W1 [V, r], W2 [r, V] are all float32 or
    all bfloat16 device tensors; anchor int32 [B]; conf_w fp32 [d + r];
    sts_T fp32 [gamma].  The call is enqueued on torch's current stream.
    Without `workspace`, a library-owned workspace cached per (device,
    stream) is used: calls on one stream share it, calls on different
    streams get different ones.  A caller-supplied workspace (zero-filled
    uint8, 256-byte aligned) must not be shared by calls that can overlap."""
    torch = _torch()
    lib = load()
    _need(U, "U")
    B, gamma, V = U.shape
    dev = U.device
    dt = U.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("U must be float32 or bfloat16")
    r = W1.shape[1]
    d = h.shape[2]
    _need(anchor, "anchor", torch.int32, (B,), dev)
    _need(h, "h", dt, (B, gamma, d), dev)
    _need(W1, "W1", dt, (V, r), dev)
    _need(W2, "W2", dt, (r, V), dev)
    _need(conf_w, "conf_w", torch.float32, (d + r,), dev)
    _need(sts_T, "sts_T", torch.float32, (gamma,), dev)
    if out is None:
        out = (torch.empty((B, gamma), dtype=torch.int32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev))
    tokens, logit, conf, surv = out
    nbytes = workspace_bytes(B, gamma, V, r)
    ws = workspace if workspace is not None else _workspace(nbytes, dev, "draft", (B, gamma))
    st = lib.dspark_markov_draft(
        B, gamma, V, r, d, DSPARK_BF16 if dt == torch.bfloat16 else DSPARK_F32,
        _ptr(anchor), _ptr(U), _ptr(h), _ptr(W1), _ptr(W2),
        _ptr(conf_w), ctypes.c_float(conf_b), _ptr(sts_T),
        DSPARK_GUMBEL if mode == "gumbel" else DSPARK_GREEDY, ctypes.c_uint64(seed & (2 ** 64 - 1)),
        _ptr(tokens), _ptr(logit), _ptr(conf), _ptr(surv),
        _ptr(ws), ctypes.c_size_t(ws.numel()), _stream())
    _check(st)
    return tokens, logit, conf, surv


def step(anchor, U, h, W1, W2, conf_w, conf_b: float, sts_T, target, t_step, n_min: int, mode: str = "greedy",
         seed: int = 0, out=None, workspace=None):
    """One step in one call (dspark_step): Markov-head drafting, the prefix
    scheduler on the drafted survivals, and verify against `target` (int32
    [B, gamma + 1]).  Returns (tokens, logit, conf, surv [B, gamma]; lens,
    accepted, bonus [B]; m [1]).  Inputs as markov_draft; t_step fp64 and
    n_min as schedule.  Without `workspace`, a library-owned workspace
    cached per (device, stream) is used."""
    torch = _torch()
    lib = load()
    _need(U, "U")
    B, gamma, V = U.shape
    dev = U.device
    dt = U.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("U must be float32 or bfloat16")
    r = W1.shape[1]
    d = h.shape[2]
    _need(anchor, "anchor", torch.int32, (B,), dev)
    _need(h, "h", dt, (B, gamma, d), dev)
    _need(W1, "W1", dt, (V, r), dev)
    _need(W2, "W2", dt, (r, V), dev)
    _need(conf_w, "conf_w", torch.float32, (d + r,), dev)
    _need(sts_T, "sts_T", torch.float32, (gamma,), dev)
    _need(target, "target", torch.int32, (B, gamma + 1), dev)
    _need(t_step, "t_step", torch.float64, None, dev)
    if out is None:
        f = lambda *sh, dtype=torch.float32: torch.empty(sh, dtype=dtype, device=dev)  # noqa: E731
        out = (f(B, gamma, dtype=torch.int32), f(B, gamma), f(B, gamma), f(B, gamma), f(B, dtype=torch.int32),
               f(B, dtype=torch.int32), f(B, dtype=torch.int32), f(1, dtype=torch.int32))
    tokens, logit, conf, surv, lens, accepted, bonus, m = out
    nbytes = int(lib.dspark_step_workspace_bytes(B, gamma, V, r))
    ws = workspace if workspace is not None else _workspace(nbytes, dev, "step", (B, gamma))
    st = lib.dspark_step(
        B, gamma, V, r, d, DSPARK_BF16 if dt == torch.bfloat16 else DSPARK_F32,
        _ptr(anchor), _ptr(U), _ptr(h), _ptr(W1), _ptr(W2), _ptr(conf_w), ctypes.c_float(conf_b), _ptr(sts_T),
        DSPARK_GUMBEL if mode == "gumbel" else DSPARK_GREEDY, ctypes.c_uint64(seed & (2 ** 64 - 1)),
        _ptr(target), _ptr(t_step), int(n_min), int(t_step.numel()),
        _ptr(tokens), _ptr(logit), _ptr(conf), _ptr(surv), _ptr(lens), _ptr(m), _ptr(accepted), _ptr(bonus),
        _ptr(ws), ctypes.c_size_t(ws.numel()), _stream())
    _check(st)
    return tokens, logit, conf, surv, lens, accepted, bonus, m


NOALLOC_SCRATCH_BYTES = 8 << 20


def markov_draft_noalloc(anchor, U, h, W1, W2, conf_w, conf_b: float, sts_T, mode: str = "greedy",
                         seed: int = 0, out=None):
    """markov_draft through dspark_markov_draft_noalloc: the library's static
    per-device scratch replaces the workspace (nothing is allocated by the
    library; `out`, if given, must hold the four output tensors).  Calls
    that can overlap on one device must not be issued."""
    torch = _torch()
    lib = load()
    _need(U, "U")
    B, gamma, V = U.shape
    dev = U.device
    dt = U.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("U must be float32 or bfloat16")
    r = W1.shape[1]
    d = h.shape[2]
    _need(anchor, "anchor", torch.int32, (B,), dev)
    _need(h, "h", dt, (B, gamma, d), dev)
    _need(W1, "W1", dt, (V, r), dev)
    _need(W2, "W2", dt, (r, V), dev)
    _need(conf_w, "conf_w", torch.float32, (d + r,), dev)
    _need(sts_T, "sts_T", torch.float32, (gamma,), dev)
    if out is None:
        out = (torch.empty((B, gamma), dtype=torch.int32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev))
    tokens, logit, conf, surv = out
    st = lib.dspark_markov_draft_noalloc(
        B, gamma, V, r, d, DSPARK_BF16 if dt == torch.bfloat16 else DSPARK_F32,
        _ptr(anchor), _ptr(U), _ptr(h), _ptr(W1), _ptr(W2),
        _ptr(conf_w), ctypes.c_float(conf_b), _ptr(sts_T),
        DSPARK_GUMBEL if mode == "gumbel" else DSPARK_GREEDY, ctypes.c_uint64(seed & (2 ** 64 - 1)),
        _ptr(tokens), _ptr(logit), _ptr(conf), _ptr(surv), _stream())
    _check(st)
    return tokens, logit, conf, surv


def rnn_workspace_bytes(B: int, gamma: int, V: int, r: int) -> int:
    return int(load().dspark_rnn_draft_workspace_bytes(B, gamma, V, r))


def rnn_draft(anchor, U, h, W1, W2, decay, conf_w, conf_b: float, sts_T, mode: str = "greedy",
              seed: int = 0, out=None, workspace=None):
    """Draft gamma tokens per request with the RNN head (recurrent state
    with per-channel decay `decay`, fp32 [r]); bfloat16 U, h, W1, W2; other
    arguments and the result as markov_draft."""
    torch = _torch()
    lib = load()
    _need(U, "U", torch.bfloat16)
    B, gamma, V = U.shape
    dev = U.device
    r = W1.shape[1]
    d = h.shape[2]
    _need(anchor, "anchor", torch.int32, (B,), dev)
    _need(h, "h", torch.bfloat16, (B, gamma, d), dev)
    _need(W1, "W1", torch.bfloat16, (V, r), dev)
    _need(W2, "W2", torch.bfloat16, (r, V), dev)
    _need(decay, "decay", torch.float32, (r,), dev)
    _need(conf_w, "conf_w", torch.float32, (d + r,), dev)
    _need(sts_T, "sts_T", torch.float32, (gamma,), dev)
    if out is None:
        out = (torch.empty((B, gamma), dtype=torch.int32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev))
    tokens, logit, conf, surv = out
    nbytes = rnn_workspace_bytes(B, gamma, V, r)
    ws = workspace if workspace is not None else _workspace(nbytes, dev, "draft", (B, gamma))
    st = lib.dspark_rnn_draft(
        B, gamma, V, r, d, DSPARK_BF16,
        _ptr(anchor), _ptr(U), _ptr(h), _ptr(W1), _ptr(W2), _ptr(decay),
        _ptr(conf_w), ctypes.c_float(conf_b), _ptr(sts_T),
        DSPARK_GUMBEL if mode == "gumbel" else DSPARK_GREEDY, ctypes.c_uint64(seed & (2 ** 64 - 1)),
        _ptr(tokens), _ptr(logit), _ptr(conf), _ptr(surv),
        _ptr(ws), ctypes.c_size_t(ws.numel()), _stream())
    _check(st)
    return tokens, logit, conf, surv


def gumbel_from_words(words, out=None):
    """The drafting kernels' Gumbel noise for given hash words (int32 device
    tensor holding the 32-bit words); returns fp32 of the same length."""
    torch = _torch()
    lib = load()
    _need(words, "words", torch.int32)
    n = words.numel()
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=words.device)
    _check(lib.dspark_gumbel_from_words(n, _ptr(words), _ptr(out), _stream()))
    return out


def parallel_draft(U, mode: str = "greedy", seed: int = 0, out=None):
    """Drafting without the sequential head: per position the arg-max of the
    base logits (or of base logits + Gumbel noise).  U [B, gamma, V] float32
    or bfloat16 device tensor; returns (tokens int32, logit fp32), [B, gamma]."""
    torch = _torch()
    lib = load()
    _need(U, "U")
    B, gamma, V = U.shape
    dev = U.device
    if U.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("U must be float32 or bfloat16")
    if out is None:
        out = (torch.empty((B, gamma), dtype=torch.int32, device=dev),
               torch.empty((B, gamma), dtype=torch.float32, device=dev))
    tokens, logit = out
    st = lib.dspark_parallel_draft(B, gamma, V, DSPARK_BF16 if U.dtype == torch.bfloat16 else DSPARK_F32, _ptr(U),
                                   DSPARK_GUMBEL if mode == "gumbel" else DSPARK_GREEDY,
                                   ctypes.c_uint64(seed & (2 ** 64 - 1)), _ptr(tokens), _ptr(logit), _stream())
    _check(st)
    return tokens, logit


def sts_fit(logit, accepted, grid, n_bins: int, out=None, workspace=None):
    """Fit the per-position confidence temperatures on a calibration set:
    logit fp32 [N, gamma] raw confidence logits, accepted int32 [N], grid
    fp32 [G] candidate temperatures.  Returns (choice int32 [gamma], T fp32
    [gamma], ece fp64 [gamma, G])."""
    torch = _torch()
    lib = load()
    _need(logit, "logit", torch.float32)
    N, gamma = logit.shape
    dev = logit.device
    _need(accepted, "accepted", torch.int32, (N,), dev)
    _need(grid, "grid", torch.float32, None, dev)
    G = grid.numel()
    if out is None:
        out = (torch.empty(gamma, dtype=torch.int32, device=dev),
               torch.empty(gamma, dtype=torch.float32, device=dev),
               torch.empty((gamma, G), dtype=torch.float64, device=dev))
    choice, T, ece = out
    nbytes = int(lib.dspark_sts_workspace_bytes(N, G, n_bins))
    ws = workspace if workspace is not None else _workspace(nbytes, dev, "sts")
    st = lib.dspark_sts_fit(N, gamma, _ptr(logit), _ptr(accepted), _ptr(grid), G, int(n_bins),
                            _ptr(choice), _ptr(T), _ptr(ece), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream())
    _check(st)
    return choice, T, ece


POLICIES = {"global": 0, "global_delayed2": 1, "threshold": 2}
LAUNCH_MODES = {"cooperative": 0, "exclusive": 1}


def set_draft_launch(mode: str) -> None:
    """Process-wide launch mode of the drafting kernel: "cooperative"
    (default) or "exclusive" (the caller guarantees that no other kernel runs
    on the device during a drafting call; saves the cooperative launch)."""
    if mode not in LAUNCH_MODES:
        raise ValueError(f"launch mode must be one of {sorted(LAUNCH_MODES)}")
    _check(load().dspark_set_draft_launch(LAUNCH_MODES[mode]))


def get_draft_launch() -> str:
    v = load().dspark_get_draft_launch()
    return {n: k for k, n in LAUNCH_MODES.items()}[v]


def schedule_threshold(surv, tau: float, out=None):
    """Static-threshold verify lengths; returns (lens int32 [B], m int32 [1])."""
    torch = _torch()
    lib = load()
    _need(surv, "surv", torch.float32)
    B, gamma = surv.shape
    dev = surv.device
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev))
    lens, m = out
    _check(lib.dspark_schedule_threshold(B, gamma, _ptr(surv), ctypes.c_float(tau), _ptr(lens), _ptr(m), _stream()))
    return lens, m


def serve(anchor0, U, h, W1, W2, conf_w, conf_b: float, sts_T, target, t_step, n_min: int,
          policy: str = "global", tau: float = 0.5, mode: str = "greedy", seed: int = 0, out=None,
          workspace=None):
    """`iters` chained draft -> schedule -> verify iterations (U [iters, B,
    gamma, V], h [iters, B, gamma, d], target int32 [iters, B, gamma + 1]).
    Returns a dict of per-iteration device tensors: tokens, logit, conf, surv
    [iters, B, gamma]; lens, accepted, bonus [iters, B]; m [iters]."""
    torch = _torch()
    lib = load()
    _need(U, "U")
    iters, B, gamma, V = U.shape
    dev = U.device
    dt = U.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("U must be float32 or bfloat16")
    r = W1.shape[1]
    d = h.shape[3]
    _need(anchor0, "anchor0", torch.int32, (B,), dev)
    _need(h, "h", dt, (iters, B, gamma, d), dev)
    _need(W1, "W1", dt, (V, r), dev)
    _need(W2, "W2", dt, (r, V), dev)
    _need(conf_w, "conf_w", torch.float32, (d + r,), dev)
    _need(sts_T, "sts_T", torch.float32, (gamma,), dev)
    _need(target, "target", torch.int32, (iters, B, gamma + 1), dev)
    _need(t_step, "t_step", torch.float64, None, dev)
    if policy not in POLICIES:
        raise ValueError(f"policy must be one of {sorted(POLICIES)}")
    if out is None:
        f = lambda *sh, dtype=torch.float32: torch.empty(sh, dtype=dtype, device=dev)  # noqa: E731
        out = dict(tokens=f(iters, B, gamma, dtype=torch.int32), logit=f(iters, B, gamma), conf=f(iters, B, gamma),
                   surv=f(iters, B, gamma), lens=f(iters, B, dtype=torch.int32),
                   accepted=f(iters, B, dtype=torch.int32), bonus=f(iters, B, dtype=torch.int32),
                   m=f(iters, dtype=torch.int32))
    nbytes = int(lib.dspark_serve_workspace_bytes(B, gamma, V, r))
    ws = workspace if workspace is not None else _workspace(nbytes, dev, "serve", (B, gamma))
    st = lib.dspark_serve(
        iters, B, gamma, V, r, d, DSPARK_BF16 if dt == torch.bfloat16 else DSPARK_F32,
        _ptr(anchor0), _ptr(U), _ptr(h), _ptr(W1), _ptr(W2), _ptr(conf_w), ctypes.c_float(conf_b), _ptr(sts_T),
        DSPARK_GUMBEL if mode == "gumbel" else DSPARK_GREEDY, ctypes.c_uint64(seed & (2 ** 64 - 1)),
        _ptr(target), _ptr(t_step), int(n_min), int(t_step.numel()), POLICIES[policy], ctypes.c_float(tau),
        _ptr(out["tokens"]), _ptr(out["logit"]), _ptr(out["conf"]), _ptr(out["surv"]), _ptr(out["lens"]),
        _ptr(out["accepted"]), _ptr(out["bonus"]), _ptr(out["m"]), _ptr(ws), ctypes.c_size_t(ws.numel()),
        _stream())
    _check(st)
    return out


def schedule_workspace_bytes(B: int, gamma: int) -> int:
    return int(load().dspark_schedule_workspace_bytes(B, gamma))


def schedule(surv, t_step, n_min: int, out=None, workspace=None, one_workgroup: bool = False):
    """Prefix scheduler; returns (lens int32 [B], m int32 [1], objective fp64 [1]).

    By default the multi-workgroup kernel runs on a library-owned workspace
    (cached per device and stream, or `workspace`, whose first 256 bytes are
    zero before the first call); `one_workgroup=True` passes no workspace and
    runs the one-workgroup sorting kernel instead."""
    torch = _torch()
    lib = load()
    _need(surv, "surv", torch.float32)
    B, gamma = surv.shape
    dev = surv.device
    _need(t_step, "t_step", torch.float64, None, dev)
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(1, dtype=torch.int32, device=dev),
               torch.empty(1, dtype=torch.float64, device=dev))
    lens, m, obj = out
    if one_workgroup:
        ws, nbytes = None, 0
    else:
        nbytes = schedule_workspace_bytes(B, gamma)
        ws = workspace if workspace is not None else (_workspace(nbytes, dev, "schedule") if nbytes else None)
    st = lib.dspark_schedule(B, gamma, _ptr(surv), _ptr(t_step), int(n_min), int(t_step.numel()),
                             _ptr(lens), _ptr(m), _ptr(obj), _ptr(ws) if ws is not None else None,
                             ws.numel() if ws is not None else 0, _stream())
    _check(st)
    return lens, m, obj


def verify(tokens, target, lens, out=None):
    """Prefix-match verify; returns (accepted int32 [B], bonus int32 [B])."""
    torch = _torch()
    lib = load()
    _need(tokens, "tokens", torch.int32)
    B, gamma = tokens.shape
    dev = tokens.device
    _need(target, "target", torch.int32, (B, gamma + 1), dev)
    _need(lens, "lens", torch.int32, (B,), dev)
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev))
    acc, bonus = out
    st = lib.dspark_verify(B, gamma, _ptr(tokens), _ptr(target), _ptr(lens),
                           _ptr(acc), _ptr(bonus), _stream())
    _check(st)
    return acc, bonus
