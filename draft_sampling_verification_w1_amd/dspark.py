"""Python binding of libdspark.so (include/dspark.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks their
dtype, shape and contiguity, and calls the entry point of the same name on
torch's current stream.  All compute happens in the HIP library; if the
library has not been built this module raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdspark.so")

F32, BF16 = 0, 1
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}

SYMBOLS = ("dspark_w2_packed_bytes", "dspark_pack_w2", "dspark_workspace_bytes",
           "dspark_draft_step", "dspark_draft_step_noalloc", "dspark_verify", "dspark_confidence", "dspark_schedule",
           "dspark_schedule_capacity", "dspark_schedule_topk", "dspark_schedule_threshold",
           "dspark_acceptance_stats", "dspark_sts_workspace_bytes", "dspark_sts_fit",
           "dspark_check_inputs", "dspark_last_error", "dspark_timing_enable",
           "dspark_timing_report")


class Problem(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int32), ("gamma", ctypes.c_int32), ("V", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


class DsparkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"dspark status {status}: {message}")
        self.status = status


_lib = None
_vp = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m draft_sampling_verification_w1_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        L.dspark_w2_packed_bytes.argtypes = [P]
        L.dspark_w2_packed_bytes.restype = ctypes.c_size_t
        L.dspark_pack_w2.argtypes = [P, _vp, _vp, _vp]
        L.dspark_workspace_bytes.argtypes = [P]
        L.dspark_workspace_bytes.restype = ctypes.c_size_t
        L.dspark_draft_step.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        ctypes.c_size_t, _vp]
        L.dspark_draft_step_noalloc.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.dspark_verify.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.dspark_confidence.argtypes = [P, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.dspark_schedule.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, _vp, ctypes.c_int32, _vp,
                                      _vp, _vp, _vp, _vp]
        L.dspark_schedule_capacity.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, _vp,
                                               ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp]
        L.dspark_schedule_topk.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp,
                                           ctypes.c_int32, _vp, _vp, _vp, _vp]
        L.dspark_schedule_threshold.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp,
                                                ctypes.c_double, _vp, _vp, _vp]
        L.dspark_acceptance_stats.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp, _vp,
                                              ctypes.c_int32, _vp, _vp, _vp, _vp, _vp]
        L.dspark_sts_workspace_bytes.argtypes = [ctypes.c_int32] * 4
        L.dspark_sts_workspace_bytes.restype = ctypes.c_size_t
        L.dspark_sts_fit.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, _vp, ctypes.c_int32, _vp,
                                     ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.dspark_check_inputs.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.dspark_last_error.restype = ctypes.c_char_p
        L.dspark_timing_enable.argtypes = [ctypes.c_int]
        L.dspark_timing_report.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
        for name in ("dspark_pack_w2", "dspark_draft_step", "dspark_draft_step_noalloc",
                     "dspark_verify", "dspark_confidence",
                     "dspark_schedule", "dspark_schedule_capacity", "dspark_schedule_topk",
                     "dspark_schedule_threshold", "dspark_acceptance_stats", "dspark_sts_fit",
                     "dspark_check_inputs",
                     "dspark_timing_enable", "dspark_timing_report"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise DsparkError(status, lib().dspark_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def problem(R: int, gamma: int, V: int, dtype: torch.dtype, seed: int, rank: int = 256) -> Problem:
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be float32 or bfloat16, got {dtype}")
    return Problem(R, gamma, V, rank, _DTYPES[dtype], 0, seed & 0xFFFFFFFFFFFFFFFF)


def w2_packed_bytes(p: Problem) -> int:
    return int(lib().dspark_w2_packed_bytes(ctypes.byref(p)))


def workspace_bytes(p: Problem) -> int:
    return int(lib().dspark_workspace_bytes(ctypes.byref(p)))


def workspace(p: Problem, device=None) -> torch.Tensor:
    n = workspace_bytes(p)
    if n == 0:
        _check(-2)
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def pack_w2(W2: torch.Tensor, V: int) -> torch.Tensor:
    """Repack W2 [256, V] once per model (dspark_pack_w2)."""
    _need(W2, "W2", shape=(256, V))
    p = problem(1, 1, V, W2.dtype, 0)
    out = torch.empty(w2_packed_bytes(p), dtype=torch.uint8, device=W2.device)
    _check(lib().dspark_pack_w2(ctypes.byref(p), _ptr(W2), _ptr(out), _stream()))
    return out


def draft_step(U, W1, W2p, anchors, seed: int, ws=None, out=None, logpd=None):
    """Stage 1 (dspark_draft_step).  U [R, gamma, V]; returns (tokens, lse, logq).
    ``logpd``: optional float32 [R, gamma, V] tensor that receives log p^d of
    every drafted position (a parity/debug output; it costs a full write)."""
    R, gamma, V = U.shape
    _need(U, "U")
    _need(W1, "W1", dtype=U.dtype, shape=(V, 256))
    _need(W2p, "W2p", dtype=torch.uint8)
    _need(anchors, "anchors", dtype=torch.int32, shape=(R,))
    p = problem(R, gamma, V, U.dtype, seed)
    if W2p.numel() < w2_packed_bytes(p):
        raise ValueError("W2p is smaller than dspark_w2_packed_bytes")
    if ws is None:
        ws = workspace(p, U.device)
    if out is None:
        out = (torch.empty((R, gamma), dtype=torch.int32, device=U.device),
               torch.empty((R, gamma), dtype=torch.float64, device=U.device),
               torch.empty((R, gamma), dtype=torch.float64, device=U.device))
    tokens, lse, logq = out
    if logpd is not None:
        _need(logpd, "logpd", dtype=torch.float32, shape=(R, gamma, V))
    _check(lib().dspark_draft_step(ctypes.byref(p), _ptr(U), _ptr(W1), _ptr(W2p), _ptr(anchors),
                                   _ptr(tokens), _ptr(lse), _ptr(logq), _ptr(logpd), _ptr(ws),
                                   ws.numel(), _stream()))
    return tokens, lse, logq


def draft_step_noalloc(U, W1, W2p, anchors, seed: int, out, logpd=None):
    """Stage 1 without a workspace (dspark_draft_step_noalloc): the library's
    fixed scratch of the current GPU serves the call.  ``out`` = (tokens int32,
    lse float64, logq float64) [R, gamma], preallocated by the caller."""
    R, gamma, V = U.shape
    _need(U, "U")
    _need(W1, "W1", dtype=U.dtype, shape=(V, 256))
    _need(W2p, "W2p", dtype=torch.uint8)
    _need(anchors, "anchors", dtype=torch.int32, shape=(R,))
    tokens, lse, logq = out
    _need(tokens, "tokens", dtype=torch.int32, shape=(R, gamma))
    _need(lse, "lse", dtype=torch.float64, shape=(R, gamma))
    _need(logq, "logq", dtype=torch.float64, shape=(R, gamma))
    if logpd is not None:
        _need(logpd, "logpd", dtype=torch.float32, shape=(R, gamma, V))
    p = problem(R, gamma, V, U.dtype, seed)
    if W2p.numel() < w2_packed_bytes(p):
        raise ValueError("W2p is smaller than dspark_w2_packed_bytes")
    _check(lib().dspark_draft_step_noalloc(ctypes.byref(p), _ptr(U), _ptr(W1), _ptr(W2p),
                                           _ptr(anchors), _ptr(tokens), _ptr(lse), _ptr(logq),
                                           _ptr(logpd), _stream()))
    return tokens, lse, logq


def timing_enable(on: bool = True):
    """Start (clearing the record) or stop per-kernel HIP-event timing."""
    _check(lib().dspark_timing_enable(1 if on else 0))


def timing_report() -> dict:
    """{kernel name: (launches, total ms)} of the recorded launches; clears the record."""
    n = lib().dspark_timing_report(None, 0)
    if n < 0:
        _check(n)
    buf = ctypes.create_string_buffer(n + 1)
    n = lib().dspark_timing_report(buf, n + 1)
    if n < 0:
        _check(n)
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out


def verify(U, W1, W2p, anchors, tokens, lse_d, logq, T, lengths, seed: int, ws=None,
           with_mask: bool = True, with_lse_t: bool = True, out=None):
    """Stage 2 (dspark_verify).  Returns dict of cstar, n_accept, out_token,
    accept_mask (optional) and lse_t (optional); ``out`` may supply that dict
    preallocated."""
    R, gamma, V = U.shape
    _need(U, "U")
    _need(T, "T", dtype=U.dtype, shape=(R, gamma + 1, V))
    _need(W1, "W1", dtype=U.dtype, shape=(V, 256))
    _need(W2p, "W2p", dtype=torch.uint8)
    _need(anchors, "anchors", dtype=torch.int32, shape=(R,))
    _need(tokens, "tokens", dtype=torch.int32, shape=(R, gamma))
    _need(lse_d, "lse_d", dtype=torch.float64, shape=(R, gamma))
    _need(logq, "logq", dtype=torch.float64, shape=(R, gamma))
    if lengths is not None:
        _need(lengths, "lengths", dtype=torch.int32, shape=(R,))
    p = problem(R, gamma, V, U.dtype, seed)
    if ws is None:
        ws = workspace(p, U.device)
    dev = U.device
    out = out if out is not None else {
        "cstar": torch.empty((R, gamma), dtype=torch.float32, device=dev),
        "n_accept": torch.empty(R, dtype=torch.int32, device=dev),
        "out_token": torch.empty(R, dtype=torch.int32, device=dev),
        "accept_mask": torch.empty((R, gamma), dtype=torch.uint8, device=dev) if with_mask else None,
        "lse_t": torch.empty((R, gamma + 1), dtype=torch.float64, device=dev) if with_lse_t else None,
    }
    _check(lib().dspark_verify(ctypes.byref(p), _ptr(U), _ptr(W1), _ptr(W2p), _ptr(anchors),
                               _ptr(tokens), _ptr(lse_d), _ptr(logq), _ptr(T), _ptr(lengths),
                               _ptr(out["cstar"]), _ptr(out["n_accept"]), _ptr(out["out_token"]),
                               _ptr(out["accept_mask"]), _ptr(out["lse_t"]), _ptr(ws), ws.numel(),
                               _stream()))
    return out


def confidence(h, w, temps, W1, anchors, tokens, seed: int = 0, out=None):
    """Confidence head with STS (dspark_confidence).  h [R, gamma, H] bf16;
    ``out`` may supply c [R, gamma] fp32 preallocated."""
    R, gamma, H = h.shape
    V = W1.shape[0]
    _need(h, "h", dtype=torch.bfloat16)
    _need(w, "w", dtype=torch.float32, shape=(H + 256,))
    _need(temps, "temps", dtype=torch.float32, shape=(gamma,))
    _need(W1, "W1", shape=(V, 256))
    _need(anchors, "anchors", dtype=torch.int32, shape=(R,))
    _need(tokens, "tokens", dtype=torch.int32, shape=(R, gamma))
    p = problem(R, gamma, V, W1.dtype, seed)
    c = torch.empty((R, gamma), dtype=torch.float32, device=h.device) if out is None else out
    _need(c, "c", dtype=torch.float32, shape=(R, gamma))
    _check(lib().dspark_confidence(ctypes.byref(p), H, _ptr(h), _ptr(w), _ptr(temps), _ptr(W1),
                                   _ptr(anchors), _ptr(tokens), _ptr(c), _stream()))
    return c


CHECK_FIELDS = ("anchors", "tokens", "U", "T", "W", "c")


def check_inputs(R: int, gamma: int, V: int, dtype, U=None, T=None, W1=None, W2=None,
                 anchors=None, tokens=None, c=None) -> dict:
    """Device-side check of the values the host cannot see (dspark_check_inputs):
    the number of anchors / tokens outside [0, V), of NaN or +inf logits in U
    and T, of non-finite weights in W1 and W2 (unpacked, [256, V]) and of
    confidences outside [0, 1].  Any tensor may be None."""
    given = [t for t in (U, T, W1, W2, anchors, tokens, c) if t is not None]
    dev = given[0].device if given else torch.device("cuda")
    for t, name, dt, shape in ((U, "U", dtype, (R, gamma, V)), (T, "T", dtype, (R, gamma + 1, V)),
                               (W1, "W1", dtype, (V, 256)), (W2, "W2", dtype, (256, V)),
                               (anchors, "anchors", torch.int32, (R,)),
                               (tokens, "tokens", torch.int32, (R, gamma)),
                               (c, "c", torch.float32, (R, gamma))):
        if t is not None:
            _need(t, name, dtype=dt, shape=shape)
    counts = torch.empty(len(CHECK_FIELDS), dtype=torch.int64, device=dev)
    p = problem(R, gamma, V, dtype, 0)
    _check(lib().dspark_check_inputs(ctypes.byref(p), _ptr(U), _ptr(T), _ptr(W1), _ptr(W2),
                                     _ptr(anchors), _ptr(tokens), _ptr(c), _ptr(counts),
                                     _stream()))
    vals = counts.cpu().tolist()
    return dict(zip(CHECK_FIELDS, vals))


def schedule(c, sps, with_path: bool = True, out=None):
    """Stages 3-4 (dspark_schedule).  c [R, gamma] fp32, sps [n] fp32; ``out``
    may supply the result dict preallocated."""
    R, gamma = c.shape
    _need(c, "c", dtype=torch.float32)
    _need(sps, "sps", dtype=torch.float32)
    dev = c.device
    if out is None:
        out = {"a": torch.empty((R, gamma), dtype=torch.float32, device=dev),
               "lengths": torch.empty(R, dtype=torch.int32, device=dev),
               "stats": torch.empty(4, dtype=torch.float64, device=dev),
               "theta_path": torch.empty(R * gamma + 1, dtype=torch.float64, device=dev)
               if with_path else None}
    _check(lib().dspark_schedule(R, gamma, _ptr(c), _ptr(sps), sps.numel(), _ptr(out["a"]),
                                 _ptr(out["lengths"]), _ptr(out["stats"]), _ptr(out["theta_path"]),
                                 _stream()))
    return out


def schedule_capacity(c, sps, with_path: bool = True):
    """Production scheduler, capacity (dspark_schedule_capacity): K = the
    candidate count with the largest Theta along the whole path (no early
    stop), left on the device in out["K"]."""
    R, gamma = c.shape
    _need(c, "c", dtype=torch.float32)
    _need(sps, "sps", dtype=torch.float32)
    dev = c.device
    out = {"a": torch.empty((R, gamma), dtype=torch.float32, device=dev),
           "K": torch.empty(1, dtype=torch.int32, device=dev),
           "lengths": torch.empty(R, dtype=torch.int32, device=dev),
           "stats": torch.empty(4, dtype=torch.float64, device=dev),
           "theta_path": torch.empty(R * gamma + 1, dtype=torch.float64, device=dev)
           if with_path else None}
    _check(lib().dspark_schedule_capacity(R, gamma, _ptr(c), _ptr(sps), sps.numel(),
                                          _ptr(out["a"]), _ptr(out["K"]), _ptr(out["lengths"]),
                                          _ptr(out["stats"]), _ptr(out["theta_path"]), _stream()))
    return out


def schedule_topk(c, K, sps):
    """Production scheduler, top-K (dspark_schedule_topk); K is a device int32
    tensor of one element."""
    R, gamma = c.shape
    _need(c, "c", dtype=torch.float32)
    _need(K, "K", dtype=torch.int32)
    _need(sps, "sps", dtype=torch.float32)
    dev = c.device
    out = {"a": torch.empty((R, gamma), dtype=torch.float32, device=dev),
           "lengths": torch.empty(R, dtype=torch.int32, device=dev),
           "stats": torch.empty(4, dtype=torch.float64, device=dev)}
    _check(lib().dspark_schedule_topk(R, gamma, _ptr(c), _ptr(K), _ptr(sps), sps.numel(),
                                      _ptr(out["a"]), _ptr(out["lengths"]), _ptr(out["stats"]),
                                      _stream()))
    return out


def schedule_threshold(c, theta: float):
    """Static-threshold verify lengths (dspark_schedule_threshold)."""
    R, gamma = c.shape
    _need(c, "c", dtype=torch.float32)
    out = {"a": torch.empty((R, gamma), dtype=torch.float32, device=c.device),
           "lengths": torch.empty(R, dtype=torch.int32, device=c.device)}
    _check(lib().dspark_schedule_threshold(R, gamma, _ptr(c), float(theta), _ptr(out["a"]),
                                           _ptr(out["lengths"]), _stream()))
    return out


def acceptance_stats(accept_mask=None, a=None, n_accept=None, thresholds=None):
    """Per-position conditional acceptance counts and a threshold sweep
    (dspark_acceptance_stats).  accept_mask [R, gamma] uint8 or None; a [R,
    gamma] fp32, n_accept [R] int32 and thresholds [n] fp64 for the sweep."""
    ref = accept_mask if accept_mask is not None else a
    R, gamma = ref.shape
    dev = ref.device
    out = {}
    if accept_mask is not None:
        _need(accept_mask, "accept_mask", dtype=torch.uint8)
        out["reached"] = torch.empty(gamma, dtype=torch.int64, device=dev)
        out["accepted"] = torch.empty(gamma, dtype=torch.int64, device=dev)
    n_thr = 0
    if thresholds is not None:
        _need(a, "a", dtype=torch.float32)
        _need(n_accept, "n_accept", dtype=torch.int32)
        _need(thresholds, "thresholds", dtype=torch.float64)
        n_thr = thresholds.numel()
        out["sweep_verified"] = torch.empty(n_thr, dtype=torch.int64, device=dev)
        out["sweep_accepted"] = torch.empty(n_thr, dtype=torch.int64, device=dev)
    _check(lib().dspark_acceptance_stats(R, gamma, _ptr(accept_mask), _ptr(a), _ptr(n_accept),
                                         _ptr(thresholds), n_thr, _ptr(out.get("reached")),
                                         _ptr(out.get("accepted")),
                                         _ptr(out.get("sweep_verified")),
                                         _ptr(out.get("sweep_accepted")), _stream()))
    return out


def sts_fit(s, y, grid, bins: int = 15):
    """Sequential Temperature Scaling fit (dspark_sts_fit).  s [N, gamma] fp64
    scores, y [N, gamma] uint8 survival labels, grid [G] fp64 temperatures."""
    N, gamma = s.shape
    _need(s, "s", dtype=torch.float64)
    _need(y, "y", dtype=torch.uint8, shape=(N, gamma))
    _need(grid, "grid", dtype=torch.float64)
    G = grid.numel()
    need = lib().dspark_sts_workspace_bytes(N, gamma, G, bins)
    if need == 0:
        raise DsparkError(-2, f"bad STS sizes N={N} gamma={gamma} G={G} bins={bins}")
    dev = s.device
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = {"temps": torch.empty(gamma, dtype=torch.float32, device=dev),
           "ece_units": torch.empty(gamma, dtype=torch.int64, device=dev),
           "ece1_units": torch.empty(gamma, dtype=torch.int64, device=dev),
           "a": torch.empty((N, gamma), dtype=torch.float32, device=dev)}
    _check(lib().dspark_sts_fit(N, gamma, _ptr(s), _ptr(y), G, _ptr(grid), bins, _ptr(out["temps"]),
                                _ptr(out["ece_units"]), _ptr(out["ece1_units"]), _ptr(out["a"]),
                                _ptr(ws), need, _stream()))
    return out
