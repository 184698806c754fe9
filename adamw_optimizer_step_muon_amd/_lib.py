"""ctypes binding of libmuonadamw.so (include/muon_adamw.h).

Argument marshalling only: tensors are checked for device, dtype and layout, their
device pointers and the current HIP stream are handed to the C ABI, and a negative
status is raised as MuonAdamWError with the library's own message.  Every step of
the optimizer runs in the library's HIP kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuonadamw.so")

MA_OK = 0
MA_ERR_INVALID_ARG = -1
MA_ERR_UNSUPPORTED = -2
MA_ERR_WORKSPACE = -3
MA_ERR_HIP = -4
MA_ERR_INTERNAL = -5
MA_MAX_NS_STEPS = 64

EXPORTED = (
    "ma_abi_version", "ma_status_string", "ma_last_error", "ma_muon_route_of",
    "ma_muon_workspace_bytes", "ma_muon_phases", "ma_muon_step", "ma_adamw_step",
    "ma_newton_schulz_workspace_bytes", "ma_newton_schulz", "ma_muon_tune", "ma_muon_tune_reset",
    "ma_adamw_step_multi", "ma_muon_check_plan", "ma_muon_ns_time", "ma_muon_static_init",
    "ma_muon_step_static", "ma_muon_tune_configs", "ma_stream_probe", "ma_mfma_probe",
)
MA_STATIC_WORKSPACE_BYTES = 512 << 20
ABI_VERSION = 4  # include/muon_adamw.h MA_ABI_VERSION


class MuonAdamWError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class _MuonBucket(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int64), ("A", ctypes.c_int64), ("B", ctypes.c_int64),
                ("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("momentum", ctypes.c_void_p)]


class _MuonHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("momentum", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("ns_eps", ctypes.c_float),
                ("nesterov", ctypes.c_int32), ("cautious_wd", ctypes.c_int32),
                ("ns_steps", ctypes.c_int32), ("scale_mode", ctypes.c_int32),
                ("ns_coeffs", ctypes.POINTER(ctypes.c_float)), ("ns_mode", ctypes.c_int32)]


class _MuonRoute(ctypes.Structure):
    _fields_ = [("transposed", ctypes.c_int32), ("m", ctypes.c_int32), ("n", ctypes.c_int32),
                ("ns_steps_run", ctypes.c_int32), ("m_pad", ctypes.c_int32),
                ("n_pad", ctypes.c_int32), ("ns_mode_run", ctypes.c_int32)]


class _GemmConfig(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int32), ("band", ctypes.c_int32), ("spread", ctypes.c_int32),
                ("pipeline", ctypes.c_int32), ("xcd", ctypes.c_int32)]


class _PlanReport(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("gemm_blocks", ctypes.c_int64),
                ("gemm_tiles", ctypes.c_int64)]


class _AdamWSegment(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("n", ctypes.c_int64)]


class _AdamWHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("step", ctypes.c_int64), ("decoupled", ctypes.c_int32),
                ("cautious_wd", ctypes.c_int32)]


@dataclass(frozen=True)
class Route:
    """Routing report of one bucket (see ma_muon_route)."""

    transposed: bool
    m: int
    n: int
    ns_steps_run: int
    m_pad: int
    n_pad: int
    ns_mode_run: int = 0


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libmuonadamw.so not found at {path}: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    lib.ma_abi_version.restype = ctypes.c_int
    # the structures below are laid out for this ABI; a library built from other sources
    # would read them wrongly
    if lib.ma_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.ma_abi_version()}, this binding "
                           f"expects {ABI_VERSION}: rebuild the library")
    lib.ma_status_string.restype = ctypes.c_char_p
    lib.ma_status_string.argtypes = [ctypes.c_int]
    lib.ma_last_error.restype = ctypes.c_char_p
    lib.ma_muon_route_of.restype = ctypes.c_int
    lib.ma_muon_route_of.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(_MuonHParams),
                                     ctypes.POINTER(_MuonRoute)]
    lib.ma_muon_workspace_bytes.restype = ctypes.c_size_t
    lib.ma_muon_workspace_bytes.argtypes = [ctypes.POINTER(_MuonBucket), ctypes.c_int32,
                                            ctypes.POINTER(_MuonHParams)]
    lib.ma_muon_phases.restype = ctypes.c_int32
    lib.ma_muon_phases.argtypes = [ctypes.POINTER(_MuonBucket), ctypes.c_int32,
                                   ctypes.POINTER(_MuonHParams), ctypes.POINTER(ctypes.c_int32)]
    lib.ma_muon_step.restype = ctypes.c_int
    lib.ma_muon_step.argtypes = [ctypes.POINTER(_MuonBucket), ctypes.c_int32,
                                 ctypes.POINTER(_MuonHParams), ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p, ctypes.POINTER(_MuonRoute)]
    lib.ma_adamw_step.restype = ctypes.c_int
    lib.ma_adamw_step.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.POINTER(_AdamWHParams), ctypes.c_void_p]
    lib.ma_newton_schulz_workspace_bytes.restype = ctypes.c_size_t
    lib.ma_newton_schulz_workspace_bytes.argtypes = [ctypes.c_int64] * 3
    lib.ma_newton_schulz.restype = ctypes.c_int
    lib.ma_newton_schulz.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int64,
                                     ctypes.POINTER(_MuonHParams), ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]
    lib.ma_muon_tune.restype = ctypes.c_int
    lib.ma_muon_tune.argtypes = [ctypes.POINTER(_MuonBucket), ctypes.c_int32,
                                 ctypes.POINTER(_MuonHParams), ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.ma_adamw_step_multi.restype = ctypes.c_int
    lib.ma_adamw_step_multi.argtypes = [ctypes.POINTER(_AdamWSegment), ctypes.c_int32,
                                        ctypes.POINTER(_AdamWHParams), ctypes.c_void_p]
    lib.ma_muon_tune_configs.restype = ctypes.c_int
    lib.ma_muon_tune_configs.argtypes = [ctypes.POINTER(_MuonBucket), ctypes.c_int32,
                                         ctypes.POINTER(_MuonHParams), ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.POINTER(_GemmConfig)]
    lib.ma_stream_probe.restype = ctypes.c_int
    lib.ma_stream_probe.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32,
                                    ctypes.c_int64, ctypes.c_void_p]
    lib.ma_mfma_probe.restype = ctypes.c_int
    lib.ma_mfma_probe.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.ma_muon_tune_reset.restype = None
    lib.ma_muon_tune_reset.argtypes = []
    lib.ma_muon_check_plan.restype = ctypes.c_int
    lib.ma_muon_check_plan.argtypes = [ctypes.POINTER(_MuonBucket), ctypes.c_int32,
                                       ctypes.POINTER(_MuonHParams), ctypes.c_int32,
                                       ctypes.POINTER(_PlanReport)]
    lib.ma_muon_static_init.restype = ctypes.c_int
    lib.ma_muon_static_init.argtypes = []
    lib.ma_muon_step_static.restype = ctypes.c_int
    lib.ma_muon_step_static.argtypes = [ctypes.POINTER(_MuonBucket), ctypes.c_int32,
                                        ctypes.POINTER(_MuonHParams), ctypes.c_void_p,
                                        ctypes.POINTER(_MuonRoute)]
    lib.ma_muon_ns_time.restype = ctypes.c_int
    lib.ma_muon_ns_time.argtypes = [ctypes.POINTER(_MuonBucket), ctypes.c_int32,
                                    ctypes.POINTER(_MuonHParams), ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_float)]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != MA_OK:
        lib = load()
        raise MuonAdamWError(status, lib.ma_last_error().decode() or
                             lib.ma_status_string(status).decode())


def abi_version() -> int:
    return load().ma_abi_version()


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _ptr(t) -> int:
    return t.data_ptr() if t is not None else 0


def _require_f32_cuda(name: str, t) -> None:
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32 (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(stream, device) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _scratch(nbytes: int, device, stream):
    """A workspace allocated for one call.  It is freed when the call returns, so when
    the kernels run on another stream than the current one it is recorded on that
    stream: the caching allocator then does not hand the memory out again before that
    stream's work is done."""
    import torch

    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        ws.record_stream(stream)
    return ws


def _muon_hparams(lr, momentum, weight_decay, nesterov, ns_steps, ns_coeffs, ns_eps,
                  cautious_wd, scale_mode, ns_mode=0):
    hp = _MuonHParams(lr=lr, momentum=momentum, weight_decay=weight_decay, ns_eps=ns_eps,
                      nesterov=int(bool(nesterov)), cautious_wd=int(bool(cautious_wd)),
                      ns_steps=int(ns_steps), scale_mode=int(scale_mode),
                      ns_mode=int(ns_mode))
    keep = None
    if ns_coeffs is not None:
        flat = [float(x) for row in ns_coeffs for x in (row if hasattr(row, "__len__") else [row])]
        if len(flat) == 3 and ns_steps != 1:
            flat = flat * int(ns_steps)  # one triple for every iteration
        if len(flat) != 3 * int(ns_steps):
            raise ValueError("ns_coeffs must be one (a, b, c) triple or ns_steps of them")
        keep = (ctypes.c_float * len(flat))(*flat)
        hp.ns_coeffs = ctypes.cast(keep, ctypes.POINTER(ctypes.c_float))
    return hp, keep


def _as_stack(t):
    """(K, A, B) view of a 3-D stack or a single 2-D matrix."""
    if t.dim() == 3:
        return t
    if t.dim() == 2:
        return t.unsqueeze(0)
    raise ValueError("Muon parameters are 2-D matrices or 3-D (K, A, B) stacks")


# --------------------------------------------------------------------------
# entry points (names of the C ABI without the ma_ prefix)
# --------------------------------------------------------------------------
def muon_route_of(A: int, B: int, ns_steps: int = 5, ns_mode: int = 0, ns_coeffs=None) -> Route:
    """The route one A x B matrix takes (ma_muon_route_of) for these steps, mode and
    coefficient table (None: the quintic)."""
    hp, _keep = _muon_hparams(0.0, 0.0, 0.0, True, int(ns_steps), ns_coeffs, 1e-7, False, 0,
                              int(ns_mode))
    out = _MuonRoute()
    _check(load().ma_muon_route_of(int(A), int(B), ctypes.byref(hp), ctypes.byref(out)))
    return Route(bool(out.transposed), out.m, out.n, out.ns_steps_run, out.m_pad, out.n_pad,
                 out.ns_mode_run)


def _bucket_array(buckets):
    arr = (_MuonBucket * max(len(buckets), 1))()
    for i, (p, g, m) in enumerate(buckets):
        K, A, B = p.shape
        arr[i] = _MuonBucket(K, A, B, _ptr(p), _ptr(g), _ptr(m))
    return arr


def _mode_hparams(ns_mode: int):
    """Hyperparameters that only carry ns_mode (for the shape-only calls)."""
    hp, _ = _muon_hparams(0.0, 0.0, 0.0, True, 5, None, 1e-7, False, 0, ns_mode)
    return hp


def muon_workspace_bytes(shapes: Sequence[Sequence[int]], ns_mode: int = 0) -> int:
    """Workspace bytes for buckets of these (K, A, B) shapes."""
    arr = (_MuonBucket * max(len(shapes), 1))()
    for i, (K, A, B) in enumerate(shapes):
        arr[i] = _MuonBucket(int(K), int(A), int(B), 0, 0, 0)
    hp = _mode_hparams(ns_mode)
    return int(load().ma_muon_workspace_bytes(arr, len(shapes), ctypes.byref(hp)))


def muon_phases(shapes: Sequence[Sequence[int]], ns_mode: int = 0):
    """(number of phases, phase index per bucket) for buckets of these (K, A, B) shapes
    (ma_muon_phases): each phase runs its own Newton-Schulz GEMM launches, 3 x ns_steps
    of them for the printed iteration."""
    n = len(shapes)
    arr = (_MuonBucket * max(n, 1))()
    for i, (K, A, B) in enumerate(shapes):
        arr[i] = _MuonBucket(int(K), int(A), int(B), 0, 0, 0)
    out = (ctypes.c_int32 * max(n, 1))()
    hp = _mode_hparams(ns_mode)
    count = int(load().ma_muon_phases(arr, n, ctypes.byref(hp), out))
    if count < 0:
        _check(count)
    return count, [int(out[i]) for i in range(n)]


def muon_tune(shapes: Sequence[Sequence[int]], *, reps: int = 3, tiles=None, workspace=None,
              stream=None, device=None, ns_mode: int = 0):
    """Per-shape Newton-Schulz GEMM tiles (ma_muon_tune) for buckets of these (K, A, B)
    shapes.  reps > 0: time the available tiles on the workspace (scratch; allocated for
    the call when None) and keep the fastest; reps == 0: pin `tiles`.  Returns the tiles
    in force, one [gram, poly, combine] list per phase."""
    import torch

    n = len(shapes)
    arr = (_MuonBucket * max(n, 1))()
    for i, (K, A, B) in enumerate(shapes):
        arr[i] = _MuonBucket(int(K), int(A), int(B), 0, 0, 0)
    hp = _mode_hparams(ns_mode)
    lib = load()
    nph, _ = muon_phases(shapes, ns_mode)
    out = (ctypes.c_int32 * max(3 * nph, 1))()
    if int(reps) == 0:
        flat = [int(t) for ph in (tiles or []) for t in ph]
        if len(flat) != 3 * nph:
            raise ValueError(f"tiles needs {nph} phases of 3 entries")
        for i, t in enumerate(flat):
            out[i] = t
        _check(lib.ma_muon_tune(arr, n, ctypes.byref(hp), None, 0, None, 0, out))
    else:
        device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        need = int(lib.ma_muon_workspace_bytes(arr, n, ctypes.byref(hp)))
        if workspace is None and need > 0:
            workspace = _scratch(need, device, stream)
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        _check(lib.ma_muon_tune(arr, n, ctypes.byref(hp), _ptr(workspace), ws_bytes,
                                _stream_handle(stream, device), int(reps), out))
    return [[int(out[3 * i + q]) for q in range(3)] for i in range(nph)]


CONFIG_KEYS = ("tile", "band", "spread", "pipeline", "xcd")
DEFAULT_CONFIG = {"tile": 0, "band": 0, "spread": -1, "pipeline": 0, "xcd": 0}


def muon_tune_configs(shapes: Sequence[Sequence[int]], *, reps: int = 3, configs=None,
                      workspace=None, stream=None, device=None, ns_mode: int = 0, grads=None):
    """Per-shape Newton-Schulz GEMM configurations (ma_muon_tune_configs) for buckets of
    these (K, A, B) shapes.  reps > 0: search tile, pipeline, band width, spreading and
    XCD order on the workspace (scratch; allocated for the call when None) and keep the
    fastest; reps == 0: pin `configs` (per phase, three dicts with keys tile, band,
    spread, pipeline, xcd; missing keys take their defaults; xcd 1 = a contiguous run of
    tiles per XCD, 2 = round-robin, 3 = the XCDs share each matrix).  grads: the buckets'
    (K, A, B) gradients, cast into the workspace before the timing so the candidates run
    on real operands.  Returns the configurations in force."""
    import torch

    n = len(shapes)
    arr = (_MuonBucket * max(n, 1))()
    for i, (K, A, B) in enumerate(shapes):
        g = 0
        if grads is not None:
            _require_f32_cuda(f"gradient {i}", grads[i])
            if tuple(_as_stack(grads[i]).shape) != (int(K), int(A), int(B)):
                raise ValueError(f"gradient {i} does not have shape {(K, A, B)}")
            g = _ptr(grads[i])
        arr[i] = _MuonBucket(int(K), int(A), int(B), 0, g, 0)
    hp = _mode_hparams(ns_mode)
    lib = load()
    nph, _ = muon_phases(shapes, ns_mode)
    out = (_GemmConfig * max(3 * nph, 1))()
    if int(reps) == 0:
        flat = [c for ph in (configs or []) for c in ph]
        if len(flat) != 3 * nph:
            raise ValueError(f"configs needs {nph} phases of 3 entries")
        for i, c in enumerate(flat):
            full = {**DEFAULT_CONFIG, **c}
            out[i] = _GemmConfig(*(int(full[k]) for k in CONFIG_KEYS))
        _check(lib.ma_muon_tune_configs(arr, n, ctypes.byref(hp), None, 0, None, 0, out))
    else:
        device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        need = int(lib.ma_muon_workspace_bytes(arr, n, ctypes.byref(hp)))
        if workspace is None and need > 0:
            workspace = _scratch(need, device, stream)
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        _check(lib.ma_muon_tune_configs(arr, n, ctypes.byref(hp), _ptr(workspace), ws_bytes,
                                        _stream_handle(stream, device), int(reps), out))
    return [[{k: int(getattr(out[3 * i + q], k)) for k in CONFIG_KEYS} for q in range(3)]
            for i in range(nph)]


def muon_static_init() -> None:
    """Resolve the current device's static workspace (ma_muon_static_init); call before
    capturing muon_step_static in a graph."""
    _check(load().ma_muon_static_init())


def muon_tune_reset() -> None:
    """Forget every tuned or pinned tile (ma_muon_tune_reset)."""
    load().ma_muon_tune_reset()


def muon_step(buckets, *, lr: float, momentum: float = 0.95, weight_decay: float = 0.0,
              nesterov: bool = True, ns_steps: int = 5, ns_coeffs=None, ns_eps: float = 1e-7,
              cautious_wd: bool = False, scale_mode: int = 0, ns_mode: int = 0, workspace=None,
              stream=None):
    """One Muon step (ma_muon_step) on (param, grad, momentum) triples of (K, A, B) or
    (A, B) fp32 GPU tensors.  ns_mode 1 runs the fp16 Gram-space iteration on buckets whose
    long side is at least 3.5x the Gram side.
    Returns the routing report of each bucket."""
    import torch

    stacks = []
    for i, (p, g, m) in enumerate(buckets):
        for name, t in (("param", p), ("grad", g), ("momentum", m)):
            _require_f32_cuda(f"bucket {i} {name}", t)
        p3, g3, m3 = _as_stack(p), _as_stack(g), _as_stack(m)
        if not (p3.shape == g3.shape == m3.shape):
            raise ValueError(f"bucket {i}: param, grad and momentum shapes differ")
        stacks.append((p3, g3, m3))
    lib = load()
    arr = _bucket_array(stacks)
    hp, _keep = _muon_hparams(lr, momentum, weight_decay, nesterov, ns_steps, ns_coeffs, ns_eps,
                              cautious_wd, scale_mode, ns_mode)
    need = int(lib.ma_muon_workspace_bytes(arr, len(stacks), ctypes.byref(hp)))
    device = stacks[0][0].device if stacks else None
    if workspace is None and need > 0:
        workspace = _scratch(need, device, stream)
    routes = (_MuonRoute * max(len(stacks), 1))()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.ma_muon_step(arr, len(stacks), ctypes.byref(hp), _ptr(workspace), ws_bytes,
                            _stream_handle(stream, device) if device is not None else 0, routes))
    return [Route(bool(r.transposed), r.m, r.n, r.ns_steps_run, r.m_pad, r.n_pad, r.ns_mode_run)
            for r in routes[:len(stacks)]]


def muon_step_static(buckets, *, lr: float, momentum: float = 0.95, weight_decay: float = 0.0,
                     nesterov: bool = True, ns_steps: int = 5, ns_coeffs=None,
                     ns_eps: float = 1e-7, cautious_wd: bool = False, scale_mode: int = 0,
                     ns_mode: int = 0, stream=None):
    """ma_muon_step on the library's static workspace (ma_muon_step_static): no device
    memory is allocated, by the library or here.  Calls on one GPU share that workspace
    and must not overlap.  Returns the routing report of each bucket."""
    stacks = []
    for i, (p, g, m) in enumerate(buckets):
        for name, t in (("param", p), ("grad", g), ("momentum", m)):
            _require_f32_cuda(f"bucket {i} {name}", t)
        p3, g3, m3 = _as_stack(p), _as_stack(g), _as_stack(m)
        if not (p3.shape == g3.shape == m3.shape):
            raise ValueError(f"bucket {i}: param, grad and momentum shapes differ")
        stacks.append((p3, g3, m3))
    arr = _bucket_array(stacks)
    hp, _keep = _muon_hparams(lr, momentum, weight_decay, nesterov, ns_steps, ns_coeffs, ns_eps,
                              cautious_wd, scale_mode, ns_mode)
    routes = (_MuonRoute * max(len(stacks), 1))()
    device = stacks[0][0].device if stacks else None
    _check(load().ma_muon_step_static(arr, len(stacks), ctypes.byref(hp),
                                      _stream_handle(stream, device) if device is not None else 0,
                                      routes))
    return [Route(bool(r.transposed), r.m, r.n, r.ns_steps_run, r.m_pad, r.n_pad, r.ns_mode_run)
            for r in routes[:len(stacks)]]


def adamw_step(param, grad, exp_avg, exp_avg_sq, *, step: int, lr: float, beta1: float = 0.9,
               beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0,
               decoupled: bool = True, cautious_wd: bool = False, stream=None) -> None:
    """One AdamW step (ma_adamw_step) over contiguous fp32 GPU tensors of equal size."""
    for name, t in (("param", param), ("grad", grad), ("exp_avg", exp_avg),
                    ("exp_avg_sq", exp_avg_sq)):
        _require_f32_cuda(name, t)
    n = param.numel()
    if not (grad.numel() == exp_avg.numel() == exp_avg_sq.numel() == n):
        raise ValueError("param, grad, exp_avg and exp_avg_sq differ in size")
    hp = _AdamWHParams(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay,
                       step=int(step), decoupled=int(bool(decoupled)),
                       cautious_wd=int(bool(cautious_wd)))
    _check(load().ma_adamw_step(_ptr(param), _ptr(grad), _ptr(exp_avg), _ptr(exp_avg_sq), n,
                                ctypes.byref(hp), _stream_handle(stream, param.device)))


def adamw_step_multi(segments, *, step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                     eps: float = 1e-8, weight_decay: float = 0.0, decoupled: bool = True,
                     cautious_wd: bool = False, stream=None) -> None:
    """One AdamW step (ma_adamw_step_multi) over (param, grad, exp_avg, exp_avg_sq) tuples of
    contiguous fp32 GPU tensors, each tuple of one size: one launch per 48 tensors."""
    segs = list(segments)
    arr = (_AdamWSegment * max(len(segs), 1))()
    device = None
    for i, (p, g, m, v) in enumerate(segs):
        for name, t in (("param", p), ("grad", g), ("exp_avg", m), ("exp_avg_sq", v)):
            _require_f32_cuda(f"segment {i} {name}", t)
        n = p.numel()
        if not (g.numel() == m.numel() == v.numel() == n):
            raise ValueError(f"segment {i}: param, grad, exp_avg and exp_avg_sq differ in size")
        arr[i] = _AdamWSegment(_ptr(p), _ptr(g), _ptr(m), _ptr(v), n)
        device = p.device
    if not segs:
        return
    hp = _AdamWHParams(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay,
                       step=int(step), decoupled=int(bool(decoupled)),
                       cautious_wd=int(bool(cautious_wd)))
    _check(load().ma_adamw_step_multi(arr, len(segs), ctypes.byref(hp),
                                      _stream_handle(stream, device)))


def newton_schulz_workspace_bytes(K: int, A: int, B: int) -> int:
    return int(load().ma_newton_schulz_workspace_bytes(int(K), int(A), int(B)))


def newton_schulz(inp, out, *, ns_steps: int = 5, ns_coeffs=None, ns_eps: float = 1e-7,
                  ns_mode: int = 0, workspace=None, stream=None) -> None:
    """The orthogonalisation alone (ma_newton_schulz): out = NS(inp), (K, A, B) or (A, B)."""
    import torch

    _require_f32_cuda("inp", inp)
    _require_f32_cuda("out", out)
    i3, o3 = _as_stack(inp), _as_stack(out)
    if i3.shape != o3.shape:
        raise ValueError("inp and out shapes differ")
    K, A, B = i3.shape
    hp, _keep = _muon_hparams(0.0, 0.0, 0.0, True, ns_steps, ns_coeffs, ns_eps, False, 0, ns_mode)
    need = newton_schulz_workspace_bytes(K, A, B)
    if workspace is None and need > 0:
        workspace = _scratch(need, inp.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().ma_newton_schulz(_ptr(i3), _ptr(o3), K, A, B, ctypes.byref(hp), _ptr(workspace),
                                   ws_bytes, _stream_handle(stream, inp.device)))


def muon_check_plan(shapes: Sequence[Sequence[int]], *, what: int = 0, ns_steps: int = 5,
                    ns_mode: int = 0, ns_coeffs=None) -> dict:
    """Dry run of the launches of ma_muon_step (what 0) or ma_newton_schulz (what 1, first
    shape) for buckets of these (K, A, B) shapes (ma_muon_check_plan): raises
    MuonAdamWError if a launch reads or writes outside its buffers or misses / repeats an
    output tile; returns the counts of what was checked."""
    n = len(shapes)
    arr = (_MuonBucket * max(n, 1))()
    for i, (K, A, B) in enumerate(shapes):
        arr[i] = _MuonBucket(int(K), int(A), int(B), 0, 0, 0)
    hp, _keep = _muon_hparams(0.02, 0.95, 0.1, True, ns_steps, ns_coeffs, 1e-7, False, 0, ns_mode)
    rep = _PlanReport()
    _check(load().ma_muon_check_plan(arr, n, ctypes.byref(hp), int(what), ctypes.byref(rep)))
    return {"launches": rep.launches, "gemm_blocks": rep.gemm_blocks, "gemm_tiles": rep.gemm_tiles}


def muon_ns_time(grads, *, reps: int = 3, ns_steps: int = 5, ns_coeffs=None, ns_eps: float = 1e-7,
                 ns_mode: int = 0, workspace=None, stream=None):
    """Milliseconds per phase of the Newton-Schulz GEMM launches of ma_muon_step on these
    (K, A, B) gradient stacks (ma_muon_ns_time; synchronises).  Each repetition first casts
    the gradients into the workspace (untimed), then times the phase's launches."""
    stacks = []
    for i, g in enumerate(grads):
        _require_f32_cuda(f"gradient {i}", g)
        stacks.append(_as_stack(g))
    n = len(stacks)
    arr = (_MuonBucket * max(n, 1))()
    for i, g in enumerate(stacks):
        K, A, B = g.shape
        arr[i] = _MuonBucket(K, A, B, 0, _ptr(g), 0)
    hp, _keep = _muon_hparams(0.0, 0.0, 0.0, True, ns_steps, ns_coeffs, ns_eps, False, 0, ns_mode)
    lib = load()
    need = int(lib.ma_muon_workspace_bytes(arr, n, ctypes.byref(hp)))
    device = stacks[0].device if stacks else None
    if workspace is None and need > 0:
        workspace = _scratch(need, device, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    nph = muon_phases([tuple(g.shape) for g in stacks], ns_mode)[0]
    out = (ctypes.c_float * max(nph, 1))()
    _check(lib.ma_muon_ns_time(arr, n, ctypes.byref(hp), _ptr(workspace), ws_bytes,
                               _stream_handle(stream, device) if device is not None else 0,
                               int(reps), out))
    return [float(out[i]) for i in range(nph)]


MFMA_PROBE_THREADS = 512
MFMA_PROBE_OPERAND_VALUES = 16 * 64 * 8


def mfma_probe_flops(blocks: int, iters: int) -> float:
    """FLOPs of one ma_mfma_probe launch: 8 waves x 8 MFMAs of 32 x 32 x 16 per round."""
    return float(blocks) * 8 * iters * 8 * 2 * 32 * 32 * 16


def mfma_probe(operands, out, iters: int, *, clocks=None, stream=None) -> None:
    """The matrix-core reference loop of ma_mfma_probe: `operands` a contiguous bf16 GPU
    tensor of at least 8192 values (16 fragments of 64 lanes x 8), `out` a contiguous fp32
    GPU tensor of blocks x 512 values (its size sets the block count), `clocks` None or a
    contiguous int64 GPU tensor of 2 x blocks values."""
    import torch

    if not (operands.is_cuda and operands.dtype == torch.bfloat16 and operands.is_contiguous()):
        raise ValueError("operands must be a contiguous bf16 GPU tensor")
    if operands.numel() < MFMA_PROBE_OPERAND_VALUES:
        raise ValueError(f"operands needs {MFMA_PROBE_OPERAND_VALUES} values")
    _require_f32_cuda("out", out)
    if out.numel() % MFMA_PROBE_THREADS:
        raise ValueError("out must hold a multiple of 512 values")
    blocks = out.numel() // MFMA_PROBE_THREADS
    if clocks is not None:
        if not (clocks.is_cuda and clocks.dtype == torch.int64 and clocks.is_contiguous()
                and clocks.numel() == 2 * blocks):
            raise ValueError("clocks must be a contiguous int64 GPU tensor of 2 x blocks values")
    _check(load().ma_mfma_probe(_ptr(operands), blocks, int(iters), _ptr(out),
                                _ptr(clocks) if clocks is not None else None,
                                _stream_handle(stream, out.device)))


def stream_probe(inputs, outputs, *, stream=None) -> None:
    """The reference stream of ma_stream_probe: reads every tensor of `inputs` (1-4) and
    writes every tensor of `outputs` (0-3), all contiguous fp32 GPU tensors of one size
    (a multiple of 4), with the AdamW kernel's access pattern and no other arithmetic."""
    ts = list(inputs) + list(outputs)
    for i, t in enumerate(ts):
        _require_f32_cuda(f"array {i}", t)
    n = ts[0].numel()
    if any(t.numel() != n for t in ts):
        raise ValueError("arrays differ in size")
    ins = (ctypes.c_void_p * 4)(*([_ptr(t) for t in inputs] + [0] * (4 - len(inputs))))
    outs = (ctypes.c_void_p * 3)(*([_ptr(t) for t in outputs] + [0] * (3 - len(outputs))))
    _check(load().ma_stream_probe(ins, len(inputs), outs, len(outputs), n,
                                  _stream_handle(stream, ts[0].device)))
