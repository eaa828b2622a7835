"""ctypes binding of libsa.so (the C ABI in include/sa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libsa.  PyTorch provides device memory and the current stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsa.so")

SA_OK, SA_E_INVALID, SA_E_UNSUPPORTED, SA_E_WORKSPACE, SA_E_HIP = range(5)
SA_BF16, SA_F32 = 0, 1
SA_FLAG_TWO_PASS, SA_FLAG_ONE_PASS = 1, 2
SA_DEVICE_ERR_OFFSETS, SA_DEVICE_ERR_EXCHANGE, SA_DEVICE_ERR_RANGE, SA_DEVICE_ERR_SKETCH_ROW = 1, 2, 4, 8
_PATH_FLAGS = {None: 0, "auto": 0, "two": SA_FLAG_TWO_PASS, "one": SA_FLAG_ONE_PASS}

# functions declared in include/sa.h
EXPORTS = ("sa_workspace_size", "sa_workspace_bytes", "sa_compress_static", "sa_compress", "sa_compress_with_events", "sa_compress_with_sbar",
           "sa_backward_workspace_size", "sa_compress_backward", "sa_compress_backward_with_events",
           "sa_compress_backward_with_sbar",
           "sa_target_attention_workspace_size", "sa_target_attention", "sa_target_attention_rows",
           "sa_cache_create", "sa_cache_destroy", "sa_cache_lookup", "sa_cache_fill_workspace_size",
           "sa_cache_fill",
           "sa_read_device_error", "sa_probe_mfma", "sa_status_string", "sa_version")
NUM_PHASE_EVENTS = 5
STATIC_SCRATCH_BYTES = 64 << 20   # SA_STATIC_SCRATCH_BYTES
NUM_BWD_PHASE_EVENTS = 6


class SaProblem(ctypes.Structure):
    _fields_ = [
        ("num_users", ctypes.c_int64),
        ("total_tokens", ctypes.c_int64),
        ("d", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class SaCacheStats(ctypes.Structure):
    _fields_ = [("hits", ctypes.c_int64), ("misses", ctypes.c_int64), ("evictions", ctypes.c_int64),
                ("expired", ctypes.c_int64)]


class SaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libsa.so (built in-tree).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    # PyTorch-ROCm ships its own HIP runtime.  Load it first so that libsa's
    # libamdhip64 dependency resolves to that same runtime: with two runtimes
    # in one process, device pointers and streams of one are invalid in the
    # other.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(p):
        raise ImportError(
            f"{p} not found: build it with `python -m prototype_attention_compression_amd.build`")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER(SaProblem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.sa_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
    lib.sa_workspace_size.restype = ctypes.c_int
    lib.sa_workspace_bytes.argtypes = [P]
    lib.sa_workspace_bytes.restype = sz
    lib.sa_compress.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sa_compress.restype = ctypes.c_int
    lib.sa_compress_static.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sa_compress_static.restype = ctypes.c_int
    lib.sa_compress_with_events.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.sa_compress_with_events.restype = ctypes.c_int
    lib.sa_compress_with_sbar.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.sa_compress_with_sbar.restype = ctypes.c_int
    lib.sa_backward_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
    lib.sa_backward_workspace_size.restype = ctypes.c_int
    lib.sa_compress_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sa_compress_backward.restype = ctypes.c_int
    lib.sa_compress_backward_with_events.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                                     vp]
    lib.sa_compress_backward_with_events.restype = ctypes.c_int
    lib.sa_compress_backward_with_sbar.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                                   vp, vp]
    lib.sa_compress_backward_with_sbar.restype = ctypes.c_int
    lib.sa_target_attention_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
    lib.sa_target_attention_workspace_size.restype = ctypes.c_int
    lib.sa_target_attention.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sa_target_attention.restype = ctypes.c_int
    lib.sa_target_attention_rows.argtypes = [P, vp, vp, vp, vp, ctypes.c_int64, vp, vp, vp, sz, vp]
    lib.sa_target_attention_rows.restype = ctypes.c_int
    i64p, i32p = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)
    lib.sa_cache_create.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double, vp, vp,
                                    ctypes.POINTER(vp)]
    lib.sa_cache_create.restype = ctypes.c_int
    lib.sa_cache_destroy.argtypes = [vp]
    lib.sa_cache_destroy.restype = ctypes.c_int
    lib.sa_cache_lookup.argtypes = [vp, i64p, ctypes.c_int64, ctypes.c_double, i32p, i64p, i32p, i64p,
                                    ctypes.POINTER(SaCacheStats)]
    lib.sa_cache_lookup.restype = ctypes.c_int
    lib.sa_cache_fill_workspace_size.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(sz)]
    lib.sa_cache_fill_workspace_size.restype = ctypes.c_int
    lib.sa_cache_fill.argtypes = [vp, P, vp, i64p, vp, vp, vp, vp, i64p, i32p, ctypes.c_int64, vp, sz, vp]
    lib.sa_cache_fill.restype = ctypes.c_int
    lib.sa_read_device_error.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int32)]
    lib.sa_read_device_error.restype = ctypes.c_int
    lib.sa_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.sa_probe_mfma.restype = ctypes.c_int
    lib.sa_status_string.argtypes = [ctypes.c_int]
    lib.sa_status_string.restype = ctypes.c_char_p
    lib.sa_version.argtypes = []
    lib.sa_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().sa_status_string(int(status)).decode()


def version() -> str:
    return load().sa_version().decode()


def problem(num_users: int, total_tokens: int, d: int, k: int, dtype: int, flags: int = 0) -> SaProblem:
    return SaProblem(int(num_users), int(total_tokens), int(d), int(k), int(dtype), int(flags))


def workspace_size(num_users: int, total_tokens: int, d: int, k: int, dtype: int = SA_BF16) -> int:
    """Bytes of device workspace sa_compress needs (pure host call)."""
    pb = problem(num_users, total_tokens, d, k, dtype)
    out = ctypes.c_size_t(0)
    st = load().sa_workspace_size(ctypes.byref(pb), ctypes.byref(out))
    if st != SA_OK:
        raise SaError(st, "sa_workspace_size")
    return int(out.value)


def backward_workspace_size(num_users: int, total_tokens: int, d: int, k: int, dtype: int = SA_BF16) -> int:
    """Bytes of device workspace sa_compress_backward needs (pure host call)."""
    pb = problem(num_users, total_tokens, d, k, dtype)
    out = ctypes.c_size_t(0)
    st = load().sa_backward_workspace_size(ctypes.byref(pb), ctypes.byref(out))
    if st != SA_OK:
        raise SaError(st, "sa_backward_workspace_size")
    return int(out.value)


def raw_compress_backward(pb: SaProblem, H, offsets, mask, Wk, Wv, P, dS, dH, dP, dWk, dWv, workspace,
                          workspace_bytes: int, stream, events=None) -> int:
    """Direct call of sa_compress_backward(_with_events); returns the status."""
    if events is None:
        return int(load().sa_compress_backward(ctypes.byref(pb), H, offsets, mask, Wk, Wv, P, dS, dH, dP, dWk,
                                               dWv, workspace, ctypes.c_size_t(workspace_bytes), stream))
    return int(load().sa_compress_backward_with_events(ctypes.byref(pb), H, offsets, mask, Wk, Wv, P, dS, dH, dP,
                                                       dWk, dWv, workspace, ctypes.c_size_t(workspace_bytes),
                                                       stream, events))


def raw_compress_backward_with_sbar(pb: SaProblem, H, offsets, mask, Wk, Wv, P, Sbar, mass, dS, dH, dP, dWk, dWv,
                                    workspace, workspace_bytes: int, stream, events=None) -> int:
    """Direct call of sa_compress_backward_with_sbar; returns the status."""
    return int(load().sa_compress_backward_with_sbar(ctypes.byref(pb), H, offsets, mask, Wk, Wv, P, Sbar, mass, dS,
                                                     dH, dP, dWk, dWv, workspace, ctypes.c_size_t(workspace_bytes),
                                                     stream, events))


def raw_compress_with_sbar(pb: SaProblem, H, offsets, mask, Wk, Wv, P, S, mass, Sbar, workspace,
                           workspace_bytes: int, stream, events=None) -> int:
    """Direct call of sa_compress_with_sbar; returns the status."""
    return int(load().sa_compress_with_sbar(ctypes.byref(pb), H, offsets, mask, Wk, Wv, P, S, mass, Sbar,
                                            workspace, ctypes.c_size_t(workspace_bytes), stream, events))


def raw_compress(pb: SaProblem, H, offsets, mask, Wk, Wv, P, S, mass, workspace,
                 workspace_bytes: int, stream, events=None) -> int:
    """Direct call with device addresses (or None); returns the status.

    ``events``: optional ctypes array of NUM_PHASE_EVENTS hipEvent_t handles.
    """
    if events is None:
        return int(load().sa_compress(ctypes.byref(pb), H, offsets, mask, Wk, Wv, P, S, mass,
                                      workspace, ctypes.c_size_t(workspace_bytes), stream))
    return int(load().sa_compress_with_events(ctypes.byref(pb), H, offsets, mask, Wk, Wv, P, S, mass,
                                              workspace, ctypes.c_size_t(workspace_bytes), stream,
                                              events))


def raw_compress_static(pb: SaProblem, H, offsets, mask, Wk, Wv, P, S, mass, device_error, stream) -> int:
    """Direct call of sa_compress_static (no workspace argument); returns the
    status."""
    return int(load().sa_compress_static(ctypes.byref(pb), H, offsets, mask, Wk, Wv, P, S, mass, device_error,
                                         stream))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def compress(H, offsets, Wk, Wv, P, mask=None, return_mass: bool = False,
             out=None, mass_out=None, workspace=None, events=None, path: Optional[str] = None,
             return_sbar: bool = False):
    """Sketches of a packed ragged batch, computed by libsa on the GPU.

    H [N, d], Wk/Wv [d, d], P [k, d]: torch tensors on the current ROCm device,
    all bfloat16 or all float32, contiguous.  offsets [R+1] int64 (device).
    mask [N] uint8/bool or None.  Returns S [R, k, d] float32 (and the masses
    [R, k] if ``return_mass``).  Runs on torch's current stream.  ``path``:
    None/"auto" (library's choice), "one" or "two" (SA_FLAG_ONE_PASS /
    SA_FLAG_TWO_PASS).  ``return_sbar`` (sa_compress_with_sbar): also return
    the mass-normalised rows Sbar [R, k, d] float32, so that the result is
    (S, mass, Sbar), the forward state ``compress_backward(sbar=, mass=)``
    takes.
    """
    import torch

    if not (H.is_cuda and offsets.is_cuda and Wk.is_cuda and Wv.is_cuda and P.is_cuda):
        raise ValueError("all tensors must be on the GPU")
    if H.dtype == torch.bfloat16:
        dt = SA_BF16
    elif H.dtype == torch.float32:
        dt = SA_F32
    else:
        raise ValueError(f"unsupported dtype {H.dtype}")
    for name, t in (("Wk", Wk), ("Wv", Wv), ("P", P)):
        if t.dtype != H.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from H dtype {H.dtype}")
    if offsets.dtype != torch.int64 or offsets.dim() != 1:
        raise ValueError("offsets must be a 1-D int64 tensor")
    if H.dim() != 2:
        raise ValueError("H must be [N, d]")
    N, d = H.shape
    k = P.shape[0]
    if Wk.shape != (d, d) or Wv.shape != (d, d) or P.shape != (k, d):
        raise ValueError("shape mismatch: need Wk, Wv [d, d] and P [k, d]")
    for name, t in (("H", H), ("Wk", Wk), ("Wv", Wv), ("P", P), ("offsets", offsets)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    R = offsets.shape[0] - 1
    if R < 0:
        raise ValueError("offsets must have at least one element")
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        if mask.dtype != torch.uint8 or mask.shape != (N,) or not mask.is_cuda or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous [N] uint8/bool GPU tensor")
    if path not in _PATH_FLAGS:
        raise ValueError(f"path must be one of {sorted(k for k in _PATH_FLAGS if k)} or None")
    dev = H.device
    pb = problem(R, N, d, k, dt, _PATH_FLAGS[path])
    wbytes = workspace_size(R, N, d, k, dt)
    if workspace is None or workspace.numel() * workspace.element_size() < wbytes:
        workspace = torch.empty(max(wbytes, 1), dtype=torch.uint8, device=dev)
    S = out if out is not None else torch.empty((R, k, d), dtype=torch.float32, device=dev)
    if S.shape != (R, k, d) or S.dtype != torch.float32 or not S.is_contiguous():
        raise ValueError("out must be a contiguous float32 [R, k, d] tensor")
    m = None
    if return_mass or return_sbar:
        m = mass_out if mass_out is not None else torch.empty((R, k), dtype=torch.float32, device=dev)
        if m.shape != (R, k) or m.dtype != torch.float32 or not m.is_contiguous():
            raise ValueError("mass_out must be a contiguous float32 [R, k] tensor")
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if return_sbar:
        Sbar = torch.empty((R, k, d), dtype=torch.float32, device=dev)
        st = raw_compress_with_sbar(pb, _ptr(H) if N > 0 else None, _ptr(offsets), _ptr(mask), _ptr(Wk),
                                    _ptr(Wv), _ptr(P), _ptr(S), _ptr(m), _ptr(Sbar), _ptr(workspace), wbytes,
                                    stream, events)
        if st != SA_OK:
            raise SaError(st, "sa_compress_with_sbar")
        return S, m, Sbar
    st = raw_compress(pb, _ptr(H) if N > 0 else None, _ptr(offsets), _ptr(mask), _ptr(Wk), _ptr(Wv),
                      _ptr(P), _ptr(S), _ptr(m), _ptr(workspace), wbytes, stream, events)
    if st != SA_OK:
        raise SaError(st, "sa_compress")
    return (S, m) if return_mass else S


PROBE_SINK_FLOATS = 131072   # SA_PROBE_SINK_FLOATS
PROBE_WAVES = 2048


def probe_mfma(operands: int, iters: int, sink, stream=None) -> float:
    """Queue sa_probe_mfma on ``stream`` (default: the current stream) and
    return the FLOP count of that launch.  ``sink``: a float32 device tensor
    of PROBE_SINK_FLOATS elements."""
    import torch

    if sink.dtype != torch.float32 or sink.numel() < PROBE_SINK_FLOATS or not sink.is_cuda:
        raise ValueError("sink: a float32 device tensor of PROBE_SINK_FLOATS elements")
    s = stream if stream is not None else torch.cuda.current_stream(sink.device)
    st = load().sa_probe_mfma(int(operands), int(iters), _ptr(sink), ctypes.c_void_p(s.cuda_stream))
    if st != SA_OK:
        raise SaError(st, "sa_probe_mfma")
    return float(PROBE_WAVES) * iters * 8 * 32768


def read_device_error(workspace) -> int:
    """Device error flag of the last sa_compress on ``workspace`` (syncs)."""
    import torch

    flag = ctypes.c_int32(0)
    stream = ctypes.c_void_p(torch.cuda.current_stream(workspace.device).cuda_stream)
    st = load().sa_read_device_error(_ptr(workspace), stream, ctypes.byref(flag))
    if st != SA_OK:
        raise SaError(st, "sa_read_device_error")
    return int(flag.value)


def compress_backward(H, offsets, Wk, Wv, P, dS, mask=None, workspace=None, events=None,
                      sbar=None, mass=None):
    """Gradients of a loss through the sketches, computed by libsa on the GPU.

    Inputs as for ``compress`` (bfloat16 only), plus dS [R, k, d] float32 =
    dLoss/dS.  Returns (dH [N, d], dP [k, d], dWk [d, d], dWv [d, d]), all
    float32; dP, dWk and dWv are summed over the users.  Runs on torch's
    current stream.  ``sbar``
    and ``mass`` (sa_compress_backward_with_sbar): the forward's Sbar
    [R, k, d] and masses [R, k] from ``compress(return_sbar=True)`` on the
    same inputs; the per-user sums are then not recomputed.
    """
    import torch

    if H.dtype != torch.bfloat16:
        raise ValueError("the backward pass is built for bfloat16 inputs")
    for name, t in (("Wk", Wk), ("Wv", Wv), ("P", P)):
        if t.dtype != H.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from H dtype {H.dtype}")
    for name, t in (("H", H), ("Wk", Wk), ("Wv", Wv), ("P", P), ("offsets", offsets), ("dS", dS)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if offsets.dtype != torch.int64 or offsets.dim() != 1 or H.dim() != 2:
        raise ValueError("offsets must be 1-D int64 and H [N, d]")
    N, d = H.shape
    k = P.shape[0]
    R = offsets.shape[0] - 1
    if Wk.shape != (d, d) or Wv.shape != (d, d) or P.shape != (k, d):
        raise ValueError("shape mismatch: need Wk, Wv [d, d] and P [k, d]")
    if dS.dtype != torch.float32 or dS.shape != (R, k, d):
        raise ValueError("dS must be float32 [R, k, d]")
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        if mask.dtype != torch.uint8 or mask.shape != (N,) or not mask.is_cuda or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous [N] uint8/bool GPU tensor")
    if (sbar is None) != (mass is None):
        raise ValueError("sbar and mass go together")
    if sbar is not None:
        if (sbar.dtype != torch.float32 or sbar.shape != (R, k, d) or mass.dtype != torch.float32
                or mass.shape != (R, k)):
            raise ValueError("sbar must be float32 [R, k, d] and mass float32 [R, k]")
        for name, t in (("sbar", sbar), ("mass", mass)):
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous GPU tensor")
    dev = H.device
    pb = problem(R, N, d, k, SA_BF16)
    wbytes = backward_workspace_size(R, N, d, k, SA_BF16)
    if workspace is None or workspace.numel() * workspace.element_size() < wbytes:
        workspace = torch.empty(max(wbytes, 1), dtype=torch.uint8, device=dev)
    dH = torch.empty((N, d), dtype=torch.float32, device=dev)
    dP = torch.empty((k, d), dtype=torch.float32, device=dev)
    dWk = torch.empty((d, d), dtype=torch.float32, device=dev)
    dWv = torch.empty((d, d), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if sbar is not None:
        st = raw_compress_backward_with_sbar(pb, _ptr(H) if N > 0 else None, _ptr(offsets), _ptr(mask), _ptr(Wk),
                                             _ptr(Wv), _ptr(P), _ptr(sbar), _ptr(mass), _ptr(dS),
                                             _ptr(dH) if N > 0 else None, _ptr(dP), _ptr(dWk), _ptr(dWv),
                                             _ptr(workspace), wbytes, stream, events)
        if st != SA_OK:
            raise SaError(st, "sa_compress_backward_with_sbar")
        return dH, dP, dWk, dWv
    st = raw_compress_backward(pb, _ptr(H) if N > 0 else None, _ptr(offsets), _ptr(mask), _ptr(Wk), _ptr(Wv),
                               _ptr(P), _ptr(dS), _ptr(dH) if N > 0 else None, _ptr(dP), _ptr(dWk), _ptr(dWv),
                               _ptr(workspace), wbytes, stream, events)
    if st != SA_OK:
        raise SaError(st, "sa_compress_backward")
    return dH, dP, dWk, dWv


def target_attention_workspace_size(num_users: int, total_candidates: int, d: int, k: int) -> int:
    """Bytes of device workspace sa_target_attention needs (pure host call)."""
    pb = problem(num_users, total_candidates, d, k, SA_BF16)
    out = ctypes.c_size_t(0)
    st = load().sa_target_attention_workspace_size(ctypes.byref(pb), ctypes.byref(out))
    if st != SA_OK:
        raise SaError(st, "sa_target_attention_workspace_size")
    return int(out.value)


def raw_target_attention(pb: SaProblem, Q, cand_offsets, S, out, lse, workspace, workspace_bytes: int,
                         stream, sketch_rows=None, sketch_count: int = 0) -> int:
    """Direct call of sa_target_attention, or of sa_target_attention_rows when
    ``sketch_rows`` is given (S then holds ``sketch_count`` sketches); returns
    the status."""
    if sketch_rows is None:
        return int(load().sa_target_attention(ctypes.byref(pb), Q, cand_offsets, S, out, lse, workspace,
                                              ctypes.c_size_t(workspace_bytes), stream))
    return int(load().sa_target_attention_rows(ctypes.byref(pb), Q, cand_offsets, S, sketch_rows,
                                               int(sketch_count), out, lse, workspace,
                                               ctypes.c_size_t(workspace_bytes), stream))


def target_attention(Q, cand_offsets, S, return_lse: bool = False, out=None, workspace=None, sketch_rows=None):
    """Sketch-branch target attention, computed by libsa on the GPU.

    Q [C, d] bfloat16 candidate queries packed user by user, cand_offsets
    [R+1] int64, S [R, k, d] float32 sketches (as ``compress`` returns).
    With ``sketch_rows`` ([R] int32 GPU tensor), user u's sketch is
    S[sketch_rows[u]] and S may hold any number of rows (e.g. a cache slab);
    an index outside S gives that user zero outputs and raises
    SA_DEVICE_ERR_SKETCH_ROW (``read_device_error(workspace)``).
    Returns out [C, d] float32 (and the natural-log normalisers [C] if
    ``return_lse``).  Runs on torch's current stream.
    """
    import torch

    if Q.dtype != torch.bfloat16 or S.dtype != torch.float32:
        raise ValueError("Q must be bfloat16 and S float32")
    for name, t in (("Q", Q), ("cand_offsets", cand_offsets), ("S", S)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if cand_offsets.dtype != torch.int64 or cand_offsets.dim() != 1 or Q.dim() != 2 or S.dim() != 3:
        raise ValueError("need Q [C, d], cand_offsets [R+1] int64, S [R, k, d]")
    C, d = Q.shape
    R = cand_offsets.shape[0] - 1
    if sketch_rows is not None:
        if (sketch_rows.dtype != torch.int32 or sketch_rows.shape != (R,) or not sketch_rows.is_cuda
                or not sketch_rows.is_contiguous()):
            raise ValueError("sketch_rows must be a contiguous [R] int32 GPU tensor")
        if S.shape[2] != d:
            raise ValueError("S must be [rows, k, d] with the candidates' d")
    elif S.shape[0] != R or S.shape[2] != d:
        raise ValueError("S must be [R, k, d] with the candidates' d and one sketch per user")
    k = S.shape[1]
    dev = Q.device
    pb = problem(R, C, d, k, SA_BF16)
    wbytes = target_attention_workspace_size(R, C, d, k)
    if workspace is None or workspace.numel() * workspace.element_size() < wbytes:
        workspace = torch.empty(max(wbytes, 1), dtype=torch.uint8, device=dev)
    o = out if out is not None else torch.empty((C, d), dtype=torch.float32, device=dev)
    if o.shape != (C, d) or o.dtype != torch.float32 or not o.is_contiguous():
        raise ValueError("out must be a contiguous float32 [C, d] tensor")
    lse = torch.empty((C,), dtype=torch.float32, device=dev) if return_lse else None
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = raw_target_attention(pb, _ptr(Q) if C > 0 else None, _ptr(cand_offsets), _ptr(S),
                              _ptr(o) if C > 0 else None, _ptr(lse) if C > 0 else None, _ptr(workspace), wbytes,
                              stream, _ptr(sketch_rows), S.shape[0])
    if st != SA_OK:
        raise SaError(st, "sa_target_attention")
    return (o, lse) if return_lse else o


class SketchCache:
    """User-keyed sketch cache over a device slab (sa_cache_* in include/sa.h).

    ``slab`` [capacity, k, d] float32 and optional ``mass_slab`` [capacity, k]
    float32 are caller-owned GPU tensors (kept referenced here).  ``lookup``
    is pure host code; ``fill`` runs the misses' compression on a stream.
    """

    def __init__(self, capacity: int, k: int, d: int, ttl_seconds: float, slab, mass_slab=None):
        import numpy as np  # noqa: F401

        self._slab, self._mass = slab, mass_slab
        self.capacity, self.k, self.d = int(capacity), int(k), int(d)
        h = ctypes.c_void_p()
        st = load().sa_cache_create(self.capacity, self.k, self.d, float(ttl_seconds), _addr(slab),
                                    _addr(mass_slab), ctypes.byref(h))
        if st != SA_OK:
            raise SaError(st, "sa_cache_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            load().sa_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def lookup(self, users, now: float):
        """Returns (slots int32 [n], miss_users int64, miss_slots int32, stats dict)."""
        import numpy as np

        u = np.ascontiguousarray(users, dtype=np.int64)
        n = u.shape[0]
        slots = np.empty(n, dtype=np.int32)
        mu = np.empty(max(n, 1), dtype=np.int64)
        ms = np.empty(max(n, 1), dtype=np.int32)
        nm = ctypes.c_int64(0)
        stats = SaCacheStats()
        st = load().sa_cache_lookup(self._h, u.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n, float(now),
                                    slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                    mu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    ms.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.byref(nm),
                                    ctypes.byref(stats))
        if st != SA_OK:
            raise SaError(st, "sa_cache_lookup")
        m = int(nm.value)
        return slots, mu[:m].copy(), ms[:m].copy(), {f: int(getattr(stats, f)) for f, _ in SaCacheStats._fields_}

    def fill(self, H_store, store_offsets_host, Wk, Wv, P, miss_users, miss_slots, mask_store=None,
             workspace=None, stream=None):
        """Compress the misses (one sa_compress launch) into their slab slots on
        ``stream`` (a torch stream; default: the current one)."""
        import numpy as np
        import torch

        mu = np.ascontiguousarray(miss_users, dtype=np.int64)
        ms = np.ascontiguousarray(miss_slots, dtype=np.int32)
        off = np.ascontiguousarray(store_offsets_host, dtype=np.int64)
        if mu.shape[0] == 0:
            return
        dt = SA_BF16 if H_store.dtype == torch.bfloat16 else SA_F32
        pb = problem(off.shape[0] - 1, int(off[-1]), self.d, self.k, dt)
        lens = off[mu + 1] - off[mu]
        need = ctypes.c_size_t(0)
        st = load().sa_cache_fill_workspace_size(ctypes.byref(pb), mu.shape[0], int(lens.sum()), ctypes.byref(need))
        if st != SA_OK:
            raise SaError(st, "sa_cache_fill_workspace_size")
        dev = H_store.device
        if workspace is None or workspace.numel() < need.value:
            workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        st = load().sa_cache_fill(self._h, ctypes.byref(pb), _addr(H_store),
                                  off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _addr(mask_store), _addr(Wk),
                                  _addr(Wv), _addr(P), mu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                  ms.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), mu.shape[0], _addr(workspace),
                                  need.value, ctypes.c_void_p(s.cuda_stream))
        if st != SA_OK:
            raise SaError(st, "sa_cache_fill")
        self._last_ws = workspace   # keep alive until the stream has used it


def _addr(t):
    """Device address of a tensor, or a plain integer address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())
