"""Thin ctypes binding of libspecverify (argument marshalling only).

Every computation happens in the HIP library; this module only checks
shapes, allocates outputs and a workspace with torch, and passes raw device
pointers plus the current HIP stream through the C ABI declared in
include/specverify.h.  If the library has not been built, loading fails
loudly: there is no CPU fallback.
"""
from __future__ import annotations

import atexit
import contextlib
import ctypes
import os
import threading
from typing import Optional, Tuple

import torch


SV_OK, SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_DTYPE, SV_ERR_WORKSPACE, SV_ERR_ALIGN, SV_ERR_HIP, SV_ERR_SCRATCH = range(8)
SV_BF16, SV_F32 = 0, 1
SV_GAVE_UP = -2   # accepted count of a request whose bounded wait gave up
SV_HOOK_CHAIN_GRID_CAP, SV_HOOK_CHAIN_SPLIT, SV_HOOK_TREE_SPLIT, SV_HOOK_SPIN_LIMIT, SV_HOOK_TREE_ALL_NODES = range(5)
SV_MAX_GAMMA = 32
SV_HINT_MAX_BATCH = 256
SV_MAX_TOPK = 128

EXPORTS = {
    # name: (restype, argtypes)
    "sv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sv_version": (ctypes.c_char_p, []),
    "sv_workspace_clear": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "sv_chain_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "sv_chain_filtered_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "spec_verify_chain": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 +
                          [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]),
    "spec_verify_chain_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 +
                                  [ctypes.c_void_p] * 3),
    "spec_verify_chain_hinted": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int] * 4 +
                                 [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]),
    "spec_verify_chain_filtered": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 4 +
                                   [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]),
    "spec_verify_chain_ragged": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int] * 4 +
                                 [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]),
    "sv_chain_topk_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "spec_verify_chain_topk": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 4 +
                               [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]),
    "sv_tree_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "spec_verify_tree": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 +
                         [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]),
    "sv_probs_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "spec_probs_debug": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 4 +
                         [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]),
    "sv_tree_mss_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "spec_verify_tree_mss": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 5 +
                             [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]),
    "spec_tree_mask": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int] +
                       [ctypes.c_void_p] * 4),
    "sv_kernel_name": (ctypes.c_char_p, [ctypes.c_int]),
    "sv_timing_begin": (ctypes.c_int, [ctypes.c_int]),
    "sv_timing_end": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int),
                                     ctypes.c_int]),
    "sv_set_test_hook": (ctypes.c_int, [ctypes.c_int, ctypes.c_longlong]),
}
SV_K_COUNT = 17

_LIB = None
_LOCK = threading.Lock()


class SVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().sv_status_string(status).decode() if _LIB is not None else str(status)
        super().__init__(f"{where}: status {status} ({msg})")


def library_path() -> str:
    """The in-tree libspecverify.so, or the build named by SV_LIBRARY (such as
    the host AddressSanitizer build of asan_build.py)."""
    return os.environ.get("SV_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                        "libspecverify.so")


def lib() -> ctypes.CDLL:
    """Load libspecverify.so (built in-tree by build.build())."""
    global _LIB
    with _LOCK:
        if _LIB is None:
            path = library_path()
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build it with "
                    "`python -m rejection_sampling_verify_15_amd.build` (no CPU fallback exists)")
            handle = ctypes.CDLL(path)
            for name, (res, args) in EXPORTS.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _LIB = handle
    return _LIB


def _check(status: int, where: str):
    if status != SV_OK:
        raise SVError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _need_cuda(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------
# workspaces: zero-filled at allocation, cached per (device, stream)
# ---------------------------------------------------------------------------
_WORKSPACES = {}


def release_workspaces() -> None:
    """Drops the cached workspaces and returns torch's cached device memory.

    Registered with atexit: it runs while the interpreter is still whole, so
    no device memory is left for torch's caching allocator to free from a
    static destructor during exit(), after tools attached to the HIP runtime
    (a profiler) may already have shut down."""
    _WORKSPACES.clear()
    try:
        if torch.cuda.is_initialized():
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    except RuntimeError:
        pass


atexit.register(release_workspaces)


@contextlib.contextmanager
def library_control(hook: int, value: int):
    """Sets one of the library's test controls (SV_HOOK_*) for the duration of
    a with-block, then restores its default.  For tests only."""
    _check(lib().sv_set_test_hook(int(hook), int(value)), "sv_set_test_hook")
    try:
        yield
    finally:
        lib().sv_set_test_hook(int(hook), 0)


def recover(out_num_accepted: torch.Tensor, ws: Optional[torch.Tensor] = None) -> bool:
    """Call once the stream is synchronised.  True if a request of the call
    reports SV_GAVE_UP: the workspace that call used (`ws`, or the cached
    workspace of the current stream when the call took the cached one) may
    then hold stale words, and it is zero-filled here, on its device's
    current stream, before anything uses it again."""
    if not bool((out_num_accepted == SV_GAVE_UP).any()):
        return False
    if ws is None:
        dev = out_num_accepted.device
        ws = _WORKSPACES.get((dev.index, torch.cuda.current_stream(dev).cuda_stream))
        if ws is None:
            return True
    stream = _stream_handle(ws.device) if ws.is_cuda else None
    _check(lib().sv_workspace_clear(_ptr(ws), ws.numel(), stream), "sv_workspace_clear")
    return True


def workspace(nbytes: int, device: torch.device) -> torch.Tensor:
    """A zero-initialised device workspace of at least nbytes for the current
    stream.  The library leaves a workspace zero-filled after every call, so
    it is reused as is; calls on one stream never overlap."""
    stream = torch.cuda.current_stream(device).cuda_stream
    key = (device.index, stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        size = max(int(nbytes), 256)
        if ws is not None:
            size = max(size, 2 * ws.numel())
        ws = torch.zeros(size, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def sampling_hint_array(hint, B: int):
    """A host byte array of the caller's expected modes (nonzero: samples),
    from a sequence, numpy array or CPU tensor of B entries; an array this
    function made is passed through, so a caller can build it once."""
    if isinstance(hint, ctypes.Array) and hint._type_ is ctypes.c_uint8:
        if len(hint) < B:
            raise ValueError(f"sampling_hint must have {B} entries")
        return hint
    if isinstance(hint, torch.Tensor):
        if hint.is_cuda:
            raise ValueError("sampling_hint must be host data: the point is to avoid reading the device")
        hint = hint.numpy()
    vals = [1 if bool(x) else 0 for x in hint]
    if len(vals) != B:
        raise ValueError(f"sampling_hint must have {B} entries")
    return (ctypes.c_uint8 * max(B, 1))(*vals)


def verify_chain(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: torch.Tensor,
                 uniforms: torch.Tensor, temperature: torch.Tensor,
                 out_tokens: Optional[torch.Tensor] = None,
                 out_num_accepted: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None,
                 sampling_hint=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """spec_verify_chain over device tensors (spec_verify_chain_hinted when
    `sampling_hint`, host data of B truth values, says which requests the
    caller expects to sample; it only changes the layout of the work).

    target [B, gamma+1, V] and draft [B, gamma, V] (bf16 or fp32, same dtype),
    draft_tokens [B, gamma] int32, uniforms [B, gamma+1] fp32,
    temperature [B] fp32.  Returns (out_tokens [B, gamma+1] int32,
    out_num_accepted [B] int32)."""
    _need_cuda(target, "target")
    if target.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V]")
    B, G1, V = target.shape
    gamma = G1 - 1
    dev = target.device
    dt = _dtype_code(target)
    if draft is not None:
        _need_cuda(draft, "draft")
        if draft.dtype != target.dtype or tuple(draft.shape) != (B, gamma, V):
            raise ValueError("draft must match target's dtype with shape [B, gamma, V]")
    for name, t, shape, dtype in (("draft_tokens", draft_tokens, (B, gamma), torch.int32),
                                  ("uniforms", uniforms, (B, gamma + 1), torch.float32),
                                  ("temperature", temperature, (B,), torch.float32)):
        _need_cuda(t, name)
        if tuple(t.shape) != shape or t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype} with shape {shape}")
    if out_tokens is None:
        out_tokens = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    if out_num_accepted is None:
        out_num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    L = lib()
    nbytes = L.sv_chain_workspace_bytes(B, gamma, V, dt)
    if ws is None:
        ws = workspace(nbytes, dev)
    if sampling_hint is not None:
        hint = sampling_hint_array(sampling_hint, B)
        st = L.spec_verify_chain_hinted(_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(uniforms),
                                        _ptr(temperature), hint, B, gamma, V, dt, _ptr(out_tokens),
                                        _ptr(out_num_accepted), _ptr(ws), ws.numel(), _stream_handle(dev))
        _check(st, "spec_verify_chain_hinted")
        return out_tokens, out_num_accepted
    st = L.spec_verify_chain(_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(uniforms),
                             _ptr(temperature), B, gamma, V, dt, _ptr(out_tokens),
                             _ptr(out_num_accepted), _ptr(ws), ws.numel(), _stream_handle(dev))
    _check(st, "spec_verify_chain")
    return out_tokens, out_num_accepted


class PreparedCall:
    """One entry point with its arguments checked and marshalled once: each
    call is the C call alone (about the cost of one kernel launch on the
    host), for loops that verify into the same device buffers step after step.
    The tensors are held, so their memory stays valid; the stream is the one
    current when the call was prepared."""

    def __init__(self, fn, name: str, args, outputs, keep):
        self._fn, self._name, self._args = fn, name, tuple(args)
        self.outputs = outputs
        self._keep = keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != SV_OK:
            raise SVError(st, self._name)
        return self.outputs


def prepare_chain(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: torch.Tensor,
                  uniforms: torch.Tensor, temperature: torch.Tensor,
                  out_tokens: Optional[torch.Tensor] = None,
                  out_num_accepted: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None, sampling_hint=None) -> PreparedCall:
    """verify_chain's checks done once: returns a PreparedCall whose every
    call runs spec_verify_chain (or spec_verify_chain_hinted) on these same
    tensors, whose contents the caller may change between calls, and returns
    (out_tokens, out_num_accepted)."""
    _need_cuda(target, "target")
    if target.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V]")
    B, G1, V = target.shape
    gamma = G1 - 1
    dev = target.device
    dt = _dtype_code(target)
    if draft is not None:
        _need_cuda(draft, "draft")
        if draft.dtype != target.dtype or tuple(draft.shape) != (B, gamma, V):
            raise ValueError("draft must match target's dtype with shape [B, gamma, V]")
    for name, t, shape, dtype in (("draft_tokens", draft_tokens, (B, gamma), torch.int32),
                                  ("uniforms", uniforms, (B, gamma + 1), torch.float32),
                                  ("temperature", temperature, (B,), torch.float32)):
        _need_cuda(t, name)
        if tuple(t.shape) != shape or t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype} with shape {shape}")
    if out_tokens is None:
        out_tokens = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    if out_num_accepted is None:
        out_num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    for name, t, shape in (("out_tokens", out_tokens, (B, gamma + 1)), ("out_num_accepted", out_num_accepted, (B,))):
        _need_cuda(t, name)
        if tuple(t.shape) != shape or t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32 with shape {shape}")
    L = lib()
    if ws is None:
        ws = workspace(L.sv_chain_workspace_bytes(B, gamma, V, dt), dev)
    head = [_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(uniforms), _ptr(temperature)]
    tail = [B, gamma, V, dt, _ptr(out_tokens), _ptr(out_num_accepted), _ptr(ws), ws.numel(), _stream_handle(dev)]
    keep = (target, draft, draft_tokens, uniforms, temperature, ws)
    if sampling_hint is not None:
        hint = sampling_hint_array(sampling_hint, B)
        return PreparedCall(L.spec_verify_chain_hinted, "spec_verify_chain_hinted", head + [hint] + tail,
                            (out_tokens, out_num_accepted), keep + (hint,))
    return PreparedCall(L.spec_verify_chain, "spec_verify_chain", head + tail, (out_tokens, out_num_accepted), keep)


def verify_chain_filtered(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: torch.Tensor,
                          uniforms: torch.Tensor, temperature: torch.Tensor,
                          top_k: Optional[torch.Tensor] = None, top_p: Optional[torch.Tensor] = None,
                          out_tokens: Optional[torch.Tensor] = None,
                          out_num_accepted: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """spec_verify_chain_filtered over device tensors: the chain call with p
    and q cut alike by top-k (top_k [B] int32) and/or top-p (top_p [B] fp32)
    over the whole vocabulary.  Shapes as verify_chain; draft is required
    when gamma > 0."""
    _need_cuda(target, "target")
    if target.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V]")
    B, G1, V = target.shape
    gamma = G1 - 1
    dev = target.device
    dt = _dtype_code(target)
    if gamma > 0:
        if draft is None:
            raise ValueError("draft is required when gamma > 0")
        _need_cuda(draft, "draft")
        if draft.dtype != target.dtype or tuple(draft.shape) != (B, gamma, V):
            raise ValueError("draft must match target's dtype with shape [B, gamma, V]")
    checks = [("draft_tokens", draft_tokens, (B, gamma), torch.int32),
              ("uniforms", uniforms, (B, gamma + 1), torch.float32),
              ("temperature", temperature, (B,), torch.float32)]
    if top_k is not None:
        checks.append(("top_k", top_k, (B,), torch.int32))
    if top_p is not None:
        checks.append(("top_p", top_p, (B,), torch.float32))
    for name, t, shape, dtype in checks:
        _need_cuda(t, name)
        if tuple(t.shape) != shape or t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype} with shape {shape}")
    if out_tokens is None:
        out_tokens = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    if out_num_accepted is None:
        out_num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    L = lib()
    if ws is None:
        ws = workspace(L.sv_chain_filtered_workspace_bytes(B, gamma, V, dt), dev)
    st = L.spec_verify_chain_filtered(_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(uniforms),
                                      _ptr(temperature), _ptr(top_k), _ptr(top_p), B, gamma, V, dt,
                                      _ptr(out_tokens), _ptr(out_num_accepted), _ptr(ws), ws.numel(),
                                      _stream_handle(dev))
    _check(st, "spec_verify_chain_filtered")
    return out_tokens, out_num_accepted


def verify_chain_noalloc(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: torch.Tensor,
                         uniforms: torch.Tensor, temperature: torch.Tensor,
                         out_tokens: torch.Tensor, out_num_accepted: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """spec_verify_chain_noalloc over device tensors: verify_chain with the
    library's static scratch array as its workspace.  The caller passes the
    outputs (out_tokens [B, gamma+1] int32, out_num_accepted [B] int32), so
    nothing is allocated on the call."""
    _need_cuda(target, "target")
    if target.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V]")
    B, G1, V = target.shape
    gamma = G1 - 1
    dev = target.device
    dt = _dtype_code(target)
    if draft is not None:
        _need_cuda(draft, "draft")
        if draft.dtype != target.dtype or tuple(draft.shape) != (B, gamma, V):
            raise ValueError("draft must match target's dtype with shape [B, gamma, V]")
    for name, t, shape, dtype in (("draft_tokens", draft_tokens, (B, gamma), torch.int32),
                                  ("uniforms", uniforms, (B, gamma + 1), torch.float32),
                                  ("temperature", temperature, (B,), torch.float32),
                                  ("out_tokens", out_tokens, (B, gamma + 1), torch.int32),
                                  ("out_num_accepted", out_num_accepted, (B,), torch.int32)):
        _need_cuda(t, name)
        if tuple(t.shape) != shape or t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype} with shape {shape}")
    st = lib().spec_verify_chain_noalloc(_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(uniforms),
                                         _ptr(temperature), B, gamma, V, dt, _ptr(out_tokens),
                                         _ptr(out_num_accepted), _stream_handle(dev))
    _check(st, "spec_verify_chain_noalloc")
    return out_tokens, out_num_accepted


def verify_chain_ragged(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: torch.Tensor,
                        uniforms: torch.Tensor, temperature: torch.Tensor,
                        gammas: Optional[torch.Tensor], want_accept_prob: bool = True,
                        ws: Optional[torch.Tensor] = None):
    """spec_verify_chain_ragged over device tensors: request b drafts
    gammas[b] tokens in arrays padded to gamma (gammas [B] int32, or None for
    all gamma).  Returns (out_tokens [B, gamma+1], out_num_accepted [B],
    accept_prob [B, gamma] float32 or None)."""
    _need_cuda(target, "target")
    if target.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V]")
    B, G1, V = target.shape
    gamma = G1 - 1
    dev = target.device
    dt = _dtype_code(target)
    if gamma > 0:
        if draft is None:
            raise ValueError("draft is required when gamma > 0")
        _need_cuda(draft, "draft")
        if draft.dtype != target.dtype or tuple(draft.shape) != (B, gamma, V):
            raise ValueError("draft must match target's dtype with shape [B, gamma, V]")
    checks = [("draft_tokens", draft_tokens, (B, gamma), torch.int32),
              ("uniforms", uniforms, (B, gamma + 1), torch.float32),
              ("temperature", temperature, (B,), torch.float32)]
    if gammas is not None:
        checks.append(("gammas", gammas, (B,), torch.int32))
    for name, t, shape, dtype in checks:
        _need_cuda(t, name)
        if tuple(t.shape) != shape or t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype} with shape {shape}")
    out_tokens = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((B,), dtype=torch.int32, device=dev)
    acc = torch.empty((B, gamma), dtype=torch.float32, device=dev) if want_accept_prob and gamma > 0 else None
    L = lib()
    nbytes = L.sv_chain_workspace_bytes(B, gamma, V, dt)
    if ws is None:
        ws = workspace(nbytes, dev)
    st = L.spec_verify_chain_ragged(_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(uniforms),
                                    _ptr(temperature), _ptr(gammas), B, gamma, V, dt, _ptr(out_tokens),
                                    _ptr(out_n), _ptr(acc), _ptr(ws), ws.numel(), _stream_handle(dev))
    _check(st, "spec_verify_chain_ragged")
    return out_tokens, out_n, acc


def verify_chain_topk(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: torch.Tensor,
                      uniforms: torch.Tensor, temperature: torch.Tensor, top_k: torch.Tensor,
                      top_p: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """spec_verify_chain_topk over device tensors: as verify_chain, with p and
    q of every sampling request filtered to their rows' top-k logits
    (top_k [B] int32), then, with top_p ([B] float32), to their top-p mass.
    Returns (out_tokens [B, gamma+1], out_num_accepted [B])."""
    _need_cuda(target, "target")
    if target.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V]")
    B, G1, V = target.shape
    gamma = G1 - 1
    dev = target.device
    dt = _dtype_code(target)
    if gamma > 0:
        if draft is None:
            raise ValueError("draft is required when gamma > 0")
        _need_cuda(draft, "draft")
        if draft.dtype != target.dtype or tuple(draft.shape) != (B, gamma, V):
            raise ValueError("draft must match target's dtype with shape [B, gamma, V]")
    for name, t, shape, dtype in (("draft_tokens", draft_tokens, (B, gamma), torch.int32),
                                  ("uniforms", uniforms, (B, gamma + 1), torch.float32),
                                  ("temperature", temperature, (B,), torch.float32),
                                  ("top_k", top_k, (B,), torch.int32),
                                  ("top_p", top_p, (B,), torch.float32)):
        if t is None and name == "top_p":
            continue
        _need_cuda(t, name)
        if tuple(t.shape) != shape or t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype} with shape {shape}")
    out_tokens = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((B,), dtype=torch.int32, device=dev)
    L = lib()
    nbytes = L.sv_chain_topk_workspace_bytes(B, gamma, V, dt)
    if ws is None:
        ws = workspace(nbytes, dev)
    st = L.spec_verify_chain_topk(_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(uniforms),
                                  _ptr(temperature), _ptr(top_k), _ptr(top_p), B, gamma, V, dt, _ptr(out_tokens),
                                  _ptr(out_n), _ptr(ws), ws.numel(), _stream_handle(dev))
    _check(st, "spec_verify_chain_topk")
    return out_tokens, out_n


def verify_tree(logits: torch.Tensor, node_tokens: torch.Tensor, parents: torch.Tensor,
                uniforms: torch.Tensor, temperature: torch.Tensor, max_depth: int,
                ws: Optional[torch.Tensor] = None):
    """spec_verify_tree over device tensors.  Returns (out_tokens, out_path_nodes,
    out_num_accepted) with shapes [B, max_depth+1], [B, max_depth+1], [B]."""
    _need_cuda(logits, "logits")
    if logits.dim() != 3:
        raise ValueError("logits must be [B, N, V]")
    B, N, V = logits.shape
    dev = logits.device
    dt = _dtype_code(logits)
    for name, t, shape, dtype in (("node_tokens", node_tokens, (B, N), torch.int32),
                                  ("parents", parents, (B, N), torch.int32),
                                  ("uniforms", uniforms, (B, N), torch.float32),
                                  ("temperature", temperature, (B,), torch.float32)):
        _need_cuda(t, name)
        if tuple(t.shape) != shape or t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype} with shape {shape}")
    out_tokens = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    out_path = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((B,), dtype=torch.int32, device=dev)
    L = lib()
    nbytes = L.sv_tree_workspace_bytes(B, N, V, dt)
    if ws is None:
        ws = workspace(nbytes, dev)
    st = L.spec_verify_tree(_ptr(logits), _ptr(node_tokens), _ptr(parents), _ptr(uniforms),
                            _ptr(temperature), B, N, V, int(max_depth), dt, _ptr(out_tokens),
                            _ptr(out_path), _ptr(out_n), _ptr(ws), ws.numel(), _stream_handle(dev))
    _check(st, "spec_verify_tree")
    return out_tokens, out_path, out_n


def verify_tree_mss(logits: torch.Tensor, draft_logits: torch.Tensor, node_tokens: torch.Tensor,
                    parents: torch.Tensor, accept_uniforms: torch.Tensor, draw_uniforms: torch.Tensor,
                    temperature: torch.Tensor, max_depth: int, ws: Optional[torch.Tensor] = None):
    """spec_verify_tree_mss over device tensors (multi-step speculative
    sampling; greedy descent for T == 0).  Returns (out_tokens, out_path_nodes,
    out_num_accepted) with shapes [B, max_depth+1], [B, max_depth+1], [B]."""
    _need_cuda(logits, "logits")
    if logits.dim() != 3:
        raise ValueError("logits must be [B, N, V]")
    B, N, V = logits.shape
    dev = logits.device
    dt = _dtype_code(logits)
    _need_cuda(draft_logits, "draft_logits")
    if draft_logits.dtype != logits.dtype or tuple(draft_logits.shape) != (B, N, V):
        raise ValueError("draft_logits must match logits' dtype and shape [B, N, V]")
    for name, t, shape, dtype in (("node_tokens", node_tokens, (B, N), torch.int32),
                                  ("parents", parents, (B, N), torch.int32),
                                  ("accept_uniforms", accept_uniforms, (B, N), torch.float32),
                                  ("draw_uniforms", draw_uniforms, (B, N), torch.float32),
                                  ("temperature", temperature, (B,), torch.float32)):
        _need_cuda(t, name)
        if tuple(t.shape) != shape or t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype} with shape {shape}")
    out_tokens = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    out_path = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((B,), dtype=torch.int32, device=dev)
    L = lib()
    nbytes = L.sv_tree_mss_workspace_bytes(B, N, V, dt)
    if ws is None:
        ws = workspace(max(int(nbytes), 256), dev)
    st = L.spec_verify_tree_mss(_ptr(logits), _ptr(draft_logits), _ptr(node_tokens), _ptr(parents),
                                _ptr(accept_uniforms), _ptr(draw_uniforms), _ptr(temperature),
                                B, N, V, int(max_depth), dt, _ptr(out_tokens), _ptr(out_path),
                                _ptr(out_n), _ptr(ws), ws.numel(), _stream_handle(dev))
    _check(st, "spec_verify_tree_mss")
    return out_tokens, out_path, out_n


def tree_mask(parents: torch.Tensor, max_depth: int, out_mask: Optional[torch.Tensor] = None,
              out_depth: Optional[torch.Tensor] = None,
              out_tree_depth: Optional[torch.Tensor] = None):
    """spec_tree_mask over device tensors.  parents [B, N] int32.  Returns
    (mask [B, N, ceil(N/64)] int64 holding the uint64 row words, depth [B, N]
    int32, tree_depth [B] int32)."""
    _need_cuda(parents, "parents")
    if parents.dim() != 2 or parents.dtype != torch.int32:
        raise ValueError("parents must be int32 with shape [B, N]")
    B, N = parents.shape
    dev = parents.device
    words = (N + 63) // 64
    if out_mask is None:
        out_mask = torch.empty((B, N, words), dtype=torch.int64, device=dev)
    if out_depth is None:
        out_depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    if out_tree_depth is None:
        out_tree_depth = torch.empty((B,), dtype=torch.int32, device=dev)
    for name, t, shape, dtype in (("out_mask", out_mask, (B, N, words), torch.int64),
                                  ("out_depth", out_depth, (B, N), torch.int32),
                                  ("out_tree_depth", out_tree_depth, (B,), torch.int32)):
        _need_cuda(t, name)
        if tuple(t.shape) != shape or t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype} with shape {shape}")
    st = lib().spec_tree_mask(_ptr(parents), B, N, int(max_depth), _ptr(out_mask), _ptr(out_depth),
                              _ptr(out_tree_depth), _stream_handle(dev))
    _check(st, "spec_tree_mask")
    return out_mask, out_depth, out_tree_depth


def probs_debug(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                temperature: torch.Tensor, ws: Optional[torch.Tensor] = None):
    """spec_probs_debug over device tensors.  Returns a dict of float32 tensors:
    p_at_draft, q_at_draft, residual_mass [B, gamma], target_lse [B, gamma+1],
    draft_lse [B, gamma]."""
    _need_cuda(target, "target")
    B, G1, V = target.shape
    gamma = G1 - 1
    dev = target.device
    dt = _dtype_code(target)
    _need_cuda(draft, "draft")
    if draft.dtype != target.dtype or tuple(draft.shape) != (B, gamma, V):
        raise ValueError("draft must match target's dtype with shape [B, gamma, V]")
    _need_cuda(draft_tokens, "draft_tokens")
    _need_cuda(temperature, "temperature")
    out = {k: torch.empty((B, gamma), dtype=torch.float32, device=dev)
           for k in ("p_at_draft", "q_at_draft", "residual_mass", "draft_lse")}
    out["target_lse"] = torch.empty((B, gamma + 1), dtype=torch.float32, device=dev)
    L = lib()
    nbytes = L.sv_probs_workspace_bytes(B, gamma, V, dt)
    if ws is None:
        ws = workspace(nbytes, dev)
    st = L.spec_probs_debug(_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(temperature),
                            B, gamma, V, dt, _ptr(out["p_at_draft"]), _ptr(out["q_at_draft"]),
                            _ptr(out["residual_mass"]), _ptr(out["target_lse"]),
                            _ptr(out["draft_lse"]), _ptr(ws), ws.numel(), _stream_handle(dev))
    _check(st, "spec_probs_debug")
    return out


# ---------------------------------------------------------------------------
# kernel timing sessions
# ---------------------------------------------------------------------------
class KernelTimer:
    """Context manager around sv_timing_begin / sv_timing_end: every kernel the
    library launches inside the block is timed by events attached to its
    dispatch.  After the block, .ms[name] and .launches[name] hold the summed
    milliseconds and launch counts per kernel."""

    def __init__(self, capacity: int):
        self.capacity = int(capacity)
        self.ms = {}
        self.launches = {}

    def __enter__(self):
        _check(lib().sv_timing_begin(self.capacity), "sv_timing_begin")
        return self

    def __exit__(self, *exc):
        L = lib()
        tot = (ctypes.c_double * SV_K_COUNT)()
        cnt = (ctypes.c_int * SV_K_COUNT)()
        st = L.sv_timing_end(tot, cnt, SV_K_COUNT)
        for k in range(SV_K_COUNT):
            if cnt[k]:
                name = L.sv_kernel_name(k).decode()
                self.ms[name] = float(tot[k])
                self.launches[name] = int(cnt[k])
        if exc[0] is None:
            _check(st, "sv_timing_end")
        return False

    def mean_us(self, name: str) -> float:
        return 1e3 * self.ms[name] / self.launches[name]
