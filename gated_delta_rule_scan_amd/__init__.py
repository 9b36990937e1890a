"""Python binding of libgdn, the MI355X gated delta-rule scan.

Argument marshalling only: every step of the scan runs in the HIP kernels of
``libgdn.so`` (built in-tree by ``gated_delta_rule_scan_amd.build``).  PyTorch
is used for device memory and the current stream.  There is no fallback: if
the library is missing, every call raises.

The C ABI (``include/gdn.h``) is mirrored name for name:
``gdn_workspace_bytes``, ``gdn_forward``, ``gdn_status_string``,
``gdn_version`` and the ``gdn_problem_t`` structure.  ``forward`` is a
convenience wrapper that allocates outputs and workspace with torch.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_OK = 0
GDN_ERR_INVALID_ARGUMENT = 1
GDN_ERR_UNSUPPORTED = 2
GDN_ERR_WORKSPACE_TOO_SMALL = 3
GDN_ERR_HIP = 4

GDN_DIR_FORWARD = 0
GDN_DIR_REVERSE = 1
GDN_DIR_BIDIRECTIONAL = 2
DIRECTIONS = {"fwd": GDN_DIR_FORWARD, "rev": GDN_DIR_REVERSE, "bi": GDN_DIR_BIDIRECTIONAL}

GDN_DTYPE_F32 = 0
GDN_DTYPE_BF16 = 1

GDN_OPT_SERIAL = 1
GDN_OPT_NO_ERASE = 2
GDN_OPT_EXCLUSIVE_FORWARD = 4
GDN_OPT_EXCLUSIVE_REVERSE = 8
GDN_OPT_TEST_NO_PREPARATION = 1 << 16  # testing only (see include/gdn.h)
# which directions read their memory before the token's own write
EXCLUSIVE = {"none": 0, "fwd": GDN_OPT_EXCLUSIVE_FORWARD, "rev": GDN_OPT_EXCLUSIVE_REVERSE,
             "both": GDN_OPT_EXCLUSIVE_FORWARD | GDN_OPT_EXCLUSIVE_REVERSE}

GDN_VDA_OPT_ADDITIVE = 1

EXPORTED = ("gdn_workspace_bytes", "gdn_forward", "gdn_forward_noalloc", "gdn_vda_workspace_bytes", "gdn_vda_forward",
            "gdn_status_string", "gdn_version")
NOALLOC_SCRATCH_BYTES = 64 << 20  # GDN_NOALLOC_SCRATCH_BYTES


class gdn_problem_t(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
        ("dk", ctypes.c_int64), ("dv", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("dv_tile", ctypes.c_int32), ("options", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("timing_events", ctypes.c_void_p),
        ("gate", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
    ]


class gdn_vda_problem_t(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
        ("dk", ctypes.c_int64), ("dv", ctypes.c_int64), ("frame", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("options", ctypes.c_int32),
        ("readout_lag", ctypes.c_int32), ("norm_eps", ctypes.c_float),
        ("gate", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("timing_events", ctypes.c_void_p),
    ]


class GdnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"libgdn: {gdn_status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgdn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gated_delta_rule_scan_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(gdn_problem_t)
        vp = ctypes.c_void_p
        L.gdn_workspace_bytes.argtypes = [P, ctypes.c_int32]
        L.gdn_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32]
        L.gdn_forward.restype = ctypes.c_int
        L.gdn_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32]
        L.gdn_forward_noalloc.restype = ctypes.c_int
        PV = ctypes.POINTER(gdn_vda_problem_t)
        L.gdn_vda_workspace_bytes.argtypes = [PV, ctypes.c_int32]
        L.gdn_vda_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_vda_forward.argtypes = [PV, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32]
        L.gdn_vda_forward.restype = ctypes.c_int
        L.gdn_status_string.argtypes = [ctypes.c_int32]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_version.argtypes = []
        L.gdn_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def gdn_workspace_bytes(problem: gdn_problem_t, direction: int) -> int:
    return int(lib().gdn_workspace_bytes(ctypes.byref(problem), int(direction)))


def gdn_forward(problem: gdn_problem_t, q: int, k: int, v: int, log_alpha: int, beta: int,
                state_in: Optional[int], state_out: Optional[int], out: int, direction: int) -> int:
    """Raw call with integer device pointers (None for NULL); returns the status."""
    return int(lib().gdn_forward(ctypes.byref(problem), q, k, v, log_alpha, beta, state_in, state_out, out,
                                 int(direction)))


def gdn_forward_noalloc(problem: gdn_problem_t, q: int, k: int, v: int, log_alpha: int, beta: int,
                        state_in: Optional[int], state_out: Optional[int], out: int, direction: int) -> int:
    """Raw call of the no-allocation entry point (the library's fixed device
    scratch replaces the workspace); returns the status."""
    return int(lib().gdn_forward_noalloc(ctypes.byref(problem), q, k, v, log_alpha, beta, state_in, state_out, out,
                                         int(direction)))


def gdn_vda_workspace_bytes(problem: gdn_vda_problem_t, direction: int) -> int:
    return int(lib().gdn_vda_workspace_bytes(ctypes.byref(problem), int(direction)))


def gdn_vda_forward(problem: gdn_vda_problem_t, q: int, k: int, v: int, log_alpha: int, beta: int,
                    state_in: Optional[int], state_out: Optional[int], out: int, direction: int) -> int:
    """Raw call of the frame-wise operator with integer device pointers; returns the status."""
    return int(lib().gdn_vda_forward(ctypes.byref(problem), q, k, v, log_alpha, beta, state_in, state_out, out,
                                     int(direction)))


def gdn_status_string(status: int) -> str:
    return lib().gdn_status_string(int(status)).decode()


def gdn_version() -> str:
    return lib().gdn_version().decode()


def _record_on(stream, tensors) -> None:
    """Tensors the binding allocated on the current stream but hands to work
    on another ``stream``: tell torch's caching allocator that ``stream`` uses
    them, so their memory is not given to new allocations until that work is
    done (the workspace and any temporary are freed when the call returns)."""
    import torch

    if stream != torch.cuda.current_stream(stream.device):
        for t in tensors:
            t.record_stream(stream)


def make_problem(B, T, H, dk, dv, dtype: int, chunk: int = 0, dv_tile: int = 0, workspace: int = 0,
                 workspace_bytes: int = 0, stream: int = 0) -> gdn_problem_t:
    return gdn_problem_t(B, T, H, dk, dv, dtype, chunk, dv_tile, 0, workspace or None, workspace_bytes,
                         stream or None, None, None, None, 0.0)


def workspace_bytes(B, T, H, dk, dv, dtype: str = "bf16", direction: str = "fwd", chunk: int = 0,
                    dv_tile: int = 0, exclusive: str = "none") -> int:
    dt = GDN_DTYPE_BF16 if dtype == "bf16" else GDN_DTYPE_F32
    prob = make_problem(B, T, H, dk, dv, dt, chunk, dv_tile)
    prob.options = EXCLUSIVE[exclusive]  # exclusive readouts on bf16 operands need more
    return gdn_workspace_bytes(prob, DIRECTIONS[direction])


def forward(q, k, v, log_alpha, beta, state_in=None, direction: str = "fwd", chunk: int = 0, dv_tile: int = 0,
            out=None, state_out=None, workspace=None, want_state: bool = True, stream=None,
            timing_events: Optional[int] = None, serial: bool = False, erase: bool = True,
            exclusive: str = "none", gate=None, norm_weight=None, norm_eps: float = 1e-6) -> Tuple:
    """Run the scan on torch CUDA tensors (layouts of include/gdn.h).

    q, k: [B,T,H,dk]; v: [B,T,H,dv] (float32 or bfloat16, same dtype);
    log_alpha, beta: [dirs,B,T,H] float32; state_in: [dirs,B,H,dv,dk] float32 or None.
    Returns (out [B,T,H,dv] float32, state_out or None).  ``state_out`` may be
    passed as the same tensor as ``state_in`` for an in-place carry.
    ``serial`` keeps both kernels on ``stream`` (GDN_OPT_SERIAL); otherwise the
    library may run the chunk preparation concurrently on its own stream.
    ``erase=False`` selects the erase-free variant (GDN_OPT_NO_ERASE: gated
    linear attention with write strength beta).
    ``exclusive``: "none", "fwd", "rev" or "both" -- the directions that read
    their memory before the token's own write, o_t = a_t S_{t-1} q^_t
    (GDN_OPT_EXCLUSIVE_FORWARD / _REVERSE): "both" makes the two scans of a
    bidirectional call cover disjoint regions, "rev" alone counts every
    token once.
    ``timing_events``: address of four caller-owned hipEvent_t (see gdn.h).
    ``gate`` [B,T,H,dv] (the type of q) with ``norm_weight`` [dv] float32: the
    readout epilogue, out = norm_weight * o / sqrt(mean_dv(o^2) + norm_eps) *
    sigmoid(gate) per (token, head).
    """
    import torch

    if exclusive not in EXCLUSIVE:
        raise ValueError(f"exclusive must be one of {sorted(EXCLUSIVE)}")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dirs = 2 if direction == "bi" else 1
    if q.dtype == torch.bfloat16:
        dt = GDN_DTYPE_BF16
    elif q.dtype == torch.float32:
        dt = GDN_DTYPE_F32
    else:
        raise TypeError("q, k, v must be float32 or bfloat16")
    for t in (q, k, v):
        if t.dtype != q.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("q, k, v must be contiguous CUDA tensors of one dtype")
    for t in (log_alpha, beta):
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (dirs, B, T, H):
            raise ValueError(f"gates must be contiguous float32 [{dirs},{B},{T},{H}]")
    if state_in is not None and (state_in.dtype != torch.float32 or not state_in.is_contiguous()
                                 or tuple(state_in.shape) != (dirs, B, H, dv, dk)):
        raise ValueError(f"state_in must be contiguous float32 [{dirs},{B},{H},{dv},{dk}]")
    dev = q.device
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    mine = []  # tensors allocated here (on the current stream)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
        mine.append(out)
    if state_out is None and want_state:
        state_out = torch.empty((dirs, B, H, dv, dk), dtype=torch.float32, device=dev)
        mine.append(state_out)
    if gate is not None:
        if gate.dtype != q.dtype or not gate.is_contiguous() or tuple(gate.shape) != (B, T, H, dv):
            raise ValueError(f"gate must be contiguous [{B},{T},{H},{dv}] of the type of q")
        if norm_weight is None or norm_weight.dtype != torch.float32 or tuple(norm_weight.shape) != (dv,):
            raise ValueError(f"norm_weight must be float32 [{dv}] when gate is given")
        if not norm_weight.is_contiguous():
            norm_weight = norm_weight.contiguous()
            mine.append(norm_weight)
    prob = make_problem(B, T, H, dk, dv, dt, chunk, dv_tile)
    prob.options = (GDN_OPT_SERIAL if serial else 0) | (0 if erase else GDN_OPT_NO_ERASE) | EXCLUSIVE[exclusive]
    if gate is not None:
        prob.gate, prob.norm_weight, prob.norm_eps = gate.data_ptr(), norm_weight.data_ptr(), norm_eps
    nbytes = gdn_workspace_bytes(prob, DIRECTIONS[direction])
    if nbytes == 0 and T > 0:
        raise GdnError(GDN_ERR_UNSUPPORTED)
    if nbytes > 0 and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        mine.append(workspace)
    _record_on(s, mine)
    prob.workspace = workspace.data_ptr() if workspace is not None else None
    prob.workspace_bytes = workspace.numel() if workspace is not None else 0
    prob.stream = s.cuda_stream
    prob.timing_events = timing_events
    st = gdn_forward(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), log_alpha.data_ptr(), beta.data_ptr(),
                     None if state_in is None else state_in.data_ptr(),
                     None if state_out is None else state_out.data_ptr(), out.data_ptr(), DIRECTIONS[direction])
    if st != GDN_OK:
        raise GdnError(st)
    return out, state_out


def vda_forward(q, k, v, log_alpha, beta, state_in=None, direction: str = "fwd", frame: int = 1560, out=None,
                state_out=None, workspace=None, want_state: bool = True, stream=None,
                timing_events: Optional[int] = None, write: str = "inverse", lag: int = 0, gate=None,
                norm_weight=None, norm_eps: float = 1e-6) -> Tuple:
    """Frame-wise delta operator on torch CUDA tensors (layouts of include/gdn.h):
    q, k [B,T,H,dk], v [B,T,H,dv]; log_alpha [dirs,B,NF,H] (one per frame of
    ``frame`` tokens); beta [dirs,B,T,H]; state_in [dirs,B,H,dv,dk] or None.
    ``write``: "inverse" (the operator) or "additive" (GDN_VDA_OPT_ADDITIVE);
    ``lag``: the readout lag in frames; ``gate`` [B,T,H,dv] (type of q) with
    ``norm_weight`` [dv] float32: the readout epilogue.
    Returns (out [B,T,H,dv] float32, state_out or None)."""
    import torch

    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dirs = 2 if direction == "bi" else 1
    NF = (T + frame - 1) // frame
    if q.dtype == torch.bfloat16:
        dt = GDN_DTYPE_BF16
    elif q.dtype == torch.float32:
        dt = GDN_DTYPE_F32
    else:
        raise TypeError("q, k, v must be float32 or bfloat16")
    for t in (q, k, v):
        if t.dtype != q.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("q, k, v must be contiguous CUDA tensors of one dtype")
    if log_alpha.dtype != torch.float32 or not log_alpha.is_contiguous() or tuple(log_alpha.shape) != (dirs, B, NF, H):
        raise ValueError(f"log_alpha must be contiguous float32 [{dirs},{B},{NF},{H}]")
    if beta.dtype != torch.float32 or not beta.is_contiguous() or tuple(beta.shape) != (dirs, B, T, H):
        raise ValueError(f"beta must be contiguous float32 [{dirs},{B},{T},{H}]")
    if state_in is not None and (state_in.dtype != torch.float32 or not state_in.is_contiguous()
                                 or tuple(state_in.shape) != (dirs, B, H, dv, dk)):
        raise ValueError(f"state_in must be contiguous float32 [{dirs},{B},{H},{dv},{dk}]")
    dev = q.device
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    mine = []  # tensors allocated here (on the current stream)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
        mine.append(out)
    if state_out is None and want_state:
        state_out = torch.empty((dirs, B, H, dv, dk), dtype=torch.float32, device=dev)
        mine.append(state_out)
    if write not in ("inverse", "additive"):
        raise ValueError("write must be 'inverse' or 'additive'")
    if gate is not None:
        if gate.dtype != q.dtype or not gate.is_contiguous() or tuple(gate.shape) != (B, T, H, dv):
            raise ValueError(f"gate must be contiguous [{B},{T},{H},{dv}] of the type of q")
        if norm_weight is None or norm_weight.dtype != torch.float32 or tuple(norm_weight.shape) != (dv,):
            raise ValueError(f"norm_weight must be float32 [{dv}] when gate is given")
        if not norm_weight.is_contiguous():
            norm_weight = norm_weight.contiguous()
            mine.append(norm_weight)
    prob = gdn_vda_problem_t(B=B, T=T, H=H, dk=dk, dv=dv, frame=frame, dtype=dt,
                             options=GDN_VDA_OPT_ADDITIVE if write == "additive" else 0, readout_lag=lag,
                             norm_eps=norm_eps, gate=None if gate is None else gate.data_ptr(),
                             norm_weight=None if gate is None else norm_weight.data_ptr())
    nbytes = gdn_vda_workspace_bytes(prob, DIRECTIONS[direction])
    if nbytes == 0 and T > 0:
        raise GdnError(GDN_ERR_UNSUPPORTED)
    if nbytes > 0 and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        mine.append(workspace)
    _record_on(s, mine)
    prob.workspace = workspace.data_ptr() if workspace is not None else None
    prob.workspace_bytes = workspace.numel() if workspace is not None else 0
    prob.stream = s.cuda_stream
    prob.timing_events = timing_events
    st = gdn_vda_forward(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), log_alpha.data_ptr(), beta.data_ptr(),
                         None if state_in is None else state_in.data_ptr(),
                         None if state_out is None else state_out.data_ptr(), out.data_ptr(), DIRECTIONS[direction])
    if st != GDN_OK:
        raise GdnError(st)
    return out, state_out


# ---- torch.library custom ops: the two calls as graph-safe operators ----
# (torch.compile traces them as opaque nodes with the output shapes below,
# instead of breaking the graph at the ctypes call)

_ops_registered = False


def register_torch_ops() -> None:
    """Register torch.ops.gdn.forward and torch.ops.gdn.vda_forward (CUDA
    tensors; outputs allocated by the op) with fake implementations for
    tracing.  Idempotent."""
    global _ops_registered
    if _ops_registered:
        return
    import torch

    @torch.library.custom_op("gdn::forward", mutates_args=(), device_types="cuda",
                             schema="(Tensor q, Tensor k, Tensor v, Tensor log_alpha, Tensor beta, Tensor? state_in, "
                                    "str direction, int chunk, int dv_tile, bool erase, str exclusive=\"none\", "
                                    "Tensor? gate=None, Tensor? norm_weight=None, float norm_eps=1e-06) "
                                    "-> (Tensor, Tensor)")
    def _forward_op(q, k, v, log_alpha, beta, state_in, direction, chunk, dv_tile, erase, exclusive="none",
                    gate=None, norm_weight=None, norm_eps=1e-6):
        return forward(q, k, v, log_alpha, beta, state_in, direction, chunk, dv_tile, erase=erase,
                       exclusive=exclusive, gate=gate, norm_weight=norm_weight, norm_eps=norm_eps)

    @_forward_op.register_fake
    def _(q, k, v, log_alpha, beta, state_in, direction, chunk, dv_tile, erase, exclusive="none", gate=None,
          norm_weight=None, norm_eps=1e-6):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        dirs = 2 if direction == "bi" else 1
        return (q.new_empty((B, T, H, dv), dtype=torch.float32),
                q.new_empty((dirs, B, H, dv, dk), dtype=torch.float32))

    @torch.library.custom_op("gdn::vda_forward", mutates_args=(), device_types="cuda",
                             schema="(Tensor q, Tensor k, Tensor v, Tensor log_alpha, Tensor beta, Tensor? state_in, "
                                    "str direction, int frame, str write, int lag, Tensor? gate, Tensor? norm_weight, "
                                    "float norm_eps) -> (Tensor, Tensor)")
    def _vda_op(q, k, v, log_alpha, beta, state_in, direction, frame, write, lag, gate, norm_weight, norm_eps):
        return vda_forward(q, k, v, log_alpha, beta, state_in, direction, frame, write=write, lag=lag, gate=gate,
                           norm_weight=norm_weight, norm_eps=norm_eps)

    @_vda_op.register_fake
    def _(q, k, v, log_alpha, beta, state_in, direction, frame, write, lag, gate, norm_weight, norm_eps):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        dirs = 2 if direction == "bi" else 1
        return (q.new_empty((B, T, H, dv), dtype=torch.float32),
                q.new_empty((dirs, B, H, dv, dk), dtype=torch.float32))

    _ops_registered = True
