"""Python binding of libmuon_ns.so — the MI355X (gfx950) Muon step.

Argument marshalling only: every stage of the step runs in the library's HIP
kernels (see ``include/muon_ns.h`` for the C ABI).  PyTorch supplies device
memory (tensors, the workspace) and the stream.  There is no CPU fallback: if
the library is not built, importing the ops raises.

Names follow the C ABI:
    muon_ns_batched(xs, outs=None, steps=5, coeffs=QUINTIC, eps=1e-7)
    muon_step(params, grads, momenta, beta=0.95, lr=0.02, steps=5, ...)
    ns_workspace_size / step_workspace_size / describe_plan
    profile_enable / profile_read
"""
from __future__ import annotations

import ctypes
import json
import os
import threading

import torch

__all__ = [
    "QUINTIC", "CUBIC", "MuonError", "lib_path", "load", "muon_ns_batched", "muon_step",
    "ns_workspace_size", "step_workspace_size", "describe_plan", "profile_enable",
    "profile_read", "abi_version", "PROFILE_KINDS", "set_tile_table", "muon_step_selected",
    "step_selected_workspace_size", "muon_ns_batched_noalloc", "NOALLOC_SCRATCH_BYTES",
    "SCALE_EXP_UNKNOWN", "scale_exp_buffer",
]

QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)

MUON_DTYPE_F32 = 0
MUON_DTYPE_BF16 = 1
ABI_VERSION = 7
NOALLOC_SCRATCH_BYTES = 64 << 20  # MUON_NOALLOC_SCRATCH_BYTES

PROFILE_KINDS = {"momentum": 0, "norm": 1, "cast": 2, "syrk": 3, "gram128": 4, "final": 5,
                 "gram256_axpy": 6, "gram256_sq": 7, "sel_accum": 8, "sel_topk": 9,
                 "sel_gather": 10, "sel_scatter": 11}

_STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "ALIAS", 4: "WORKSPACE",
           5: "HIP", 6: "NO_DEVICE"}

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libmuon_ns.so")


class MuonError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.status_name = _STATUS.get(status, str(status))


class MuonNsDesc(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("out", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ld_x", ctypes.c_int64), ("ld_out", ctypes.c_int64)]


class MuonTileEntry(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("op", ctypes.c_int32),
                ("count_class", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("xcd_window", ctypes.c_int32), ("band", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class MuonStepOpts(ctypes.Structure):
    _fields_ = [("nesterov", ctypes.c_int32), ("weight_decay", ctypes.c_float),
                ("grad_dtype", ctypes.c_int32), ("overlap", ctypes.c_int32),
                ("max_workspace_bytes", ctypes.c_uint64), ("scale_exp", ctypes.c_void_p)]


# muon_step_opts_t.scale_exp entry that carries no exponent (INT32_MIN)
SCALE_EXP_UNKNOWN = -2**31


def scale_exp_buffer(n: int, device) -> torch.Tensor:
    """A fresh carried-exponent buffer for muon_step(scale_exp=...): n int32
    entries on `device`, all unknown."""
    return torch.full((n,), SCALE_EXP_UNKNOWN, dtype=torch.int32, device=device)


_lib = None
_lock = threading.Lock()


def load():
    """Load the HIP library (torch is imported first so that the library binds
    to the HIP runtime torch already uses)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is not built; run `python -m muon_newton_schulz_06_amd.build` "
                "(or __graft_entry__.build()) first — there is no CPU fallback")
        L = ctypes.CDLL(path)
        vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                 ctypes.c_float, ctypes.c_size_t)
        L.muon_abi_version.restype = i32
        L.muon_last_error.restype = ctypes.c_char_p
        L.muon_ns_batched.argtypes = [ctypes.POINTER(MuonNsDesc), i32, i32, ctypes.POINTER(f32),
                                      i32, f32, vp, sz, vp]
        L.muon_ns_batched.restype = i32
        L.muon_ns_batched_noalloc.argtypes = [ctypes.POINTER(MuonNsDesc), i32, i32,
                                              ctypes.POINTER(f32), i32, f32, vp]
        L.muon_ns_batched_noalloc.restype = i32
        L.muon_ns_workspace_size.argtypes = [ctypes.POINTER(MuonNsDesc), i32, i32,
                                             ctypes.POINTER(sz)]
        L.muon_ns_workspace_size.restype = i32
        L.muon_step.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                ctypes.POINTER(i64), ctypes.POINTER(i64), i32, i32, f32, f32, i32,
                                ctypes.POINTER(f32), f32, vp, sz, vp]
        L.muon_step.restype = i32
        L.muon_step_ex.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                   ctypes.POINTER(i64), ctypes.POINTER(i64), i32, i32, f32, f32,
                                   i32, ctypes.POINTER(f32), f32, ctypes.POINTER(MuonStepOpts),
                                   vp, sz, vp]
        L.muon_step_ex.restype = i32
        L.muon_step_workspace_size.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(i64), i32,
                                               ctypes.POINTER(sz)]
        L.muon_step_workspace_size.restype = i32
        L.muon_step_selected.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                         ctypes.POINTER(i64), ctypes.POINTER(i64), i32, i32, f32,
                                         f32, i32, ctypes.POINTER(f32), f32, ctypes.c_double, vp,
                                         sz, vp]
        L.muon_step_selected.restype = i32
        L.muon_step_selected_workspace_size.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(i64),
                                                        i32, ctypes.c_double, ctypes.POINTER(sz)]
        L.muon_step_selected_workspace_size.restype = i32
        L.muon_describe_plan.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(i64), i32, i32, i32,
                                         i32, ctypes.POINTER(f32), ctypes.c_char_p, sz]
        L.muon_describe_plan.restype = i32
        L.muon_set_tile_table.argtypes = [ctypes.POINTER(MuonTileEntry), i32]
        L.muon_set_tile_table.restype = i32
        L.muon_profile_enable.argtypes = [i32]
        L.muon_profile_enable.restype = i32
        L.muon_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)]
        L.muon_profile_read.restype = i32
        if L.muon_abi_version() != ABI_VERSION:
            raise ImportError(f"libmuon_ns ABI {L.muon_abi_version()} != {ABI_VERSION}")
        _lib = L
        return L


def _check(status: int):
    if status != 0:
        raise MuonError(status, load().muon_last_error().decode())


def abi_version() -> int:
    return int(load().muon_abi_version())


def _coeffs(c):
    return (ctypes.c_float * 3)(*[float(v) for v in c])


def _dtype_code(dt) -> int:
    if dt == torch.float32:
        return MUON_DTYPE_F32
    if dt == torch.bfloat16:
        return MUON_DTYPE_BF16
    raise TypeError(f"unsupported dtype {dt}; use float32 or bfloat16")


def _stream_handle(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


_ws_cache: dict = {}
_ws_lock = threading.Lock()


def _workspace(nbytes: int, device, user, stream=None):
    """The workspace of a call: the caller's buffer, or a cached one.

    Cached buffers are kept per (device, stream) and allocated while that
    stream is current, so the caching allocator files them under the stream
    the library's kernels use: calls on one stream reuse its buffer in stream
    order, calls on different streams never share one, and a buffer dropped
    for a larger one is only handed out again for work on that same stream
    (after the kernels already enqueued there)."""
    if nbytes == 0:
        return None, 0
    if user is not None:
        if user.device != device:
            raise ValueError("workspace on another device")
        return user, user.numel() * user.element_size()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    key = (device.type, device.index, s.cuda_stream)
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            _ws_cache.pop(key, None)
            with torch.cuda.stream(s):
                buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
            _ws_cache[key] = buf
    return buf, buf.numel()


def release_workspace():
    """Drop the cached workspace buffers (the next call allocates anew)."""
    with _ws_lock:
        _ws_cache.clear()


def _mat_fields(t: torch.Tensor):
    """(address or 0, rows, cols, row stride in elements) of a 2-D matrix
    whose rows are contiguous; strides of size-1 dimensions carry no
    information and are ignored, an empty matrix gets max(cols, 1).  Few
    tensor accesses: for calls of many small matrices the binding's cost is
    mostly this."""
    if t.dim() != 2:
        raise ValueError("matrices must be 2-D")
    rows, cols = t.shape
    if rows == 0 or cols == 0:
        return 0, rows, cols, max(cols, 1)
    s0, s1 = t.stride()
    if cols > 1 and s1 != 1:
        raise ValueError("matrix rows must be contiguous (stride(1) == 1)")
    ld = s0 if rows > 1 else cols
    if ld < cols:
        raise ValueError("row stride smaller than the row length")
    return t.data_ptr(), rows, cols, ld


def _same_device_dtype(xs, outs):
    """The one CUDA/HIP device and dtype of every x and out (ValueError /
    TypeError otherwise), with matching shapes."""
    dev, dt = xs[0].device, xs[0].dtype
    if dev.type != "cuda" or {t.device for t in xs} != {dev} or {t.device for t in outs} != {dev}:
        raise ValueError("all tensors must be on one CUDA/HIP device")
    if {t.dtype for t in xs} != {dt} or {t.dtype for t in outs} != {dt}:
        raise TypeError("all tensors must share one dtype")
    if any(x.shape != o.shape for x, o in zip(xs, outs)):
        raise ValueError("out shape differs from x shape")
    return dev, dt


def _ns_descs(xs, outs):
    """muon_ns_desc_t array (six 8-byte fields per matrix), filled in one
    ctypes construction from a flat list."""
    flat = []
    for x, o in zip(xs, outs):
        px, r, c, lx = _mat_fields(x)
        po, _, _, lo = _mat_fields(o)
        flat += (px, po, r, c, lx, lo)
    n = max(len(xs), 1)
    buf = (ctypes.c_int64 * (6 * n))(*flat)
    return (MuonNsDesc * n).from_buffer(buf)


def ns_workspace_size(shapes, dtype=torch.bfloat16) -> int:
    L = load()
    arr = (MuonNsDesc * max(len(shapes), 1))()
    for i, (r, c) in enumerate(shapes):
        arr[i].rows, arr[i].cols, arr[i].ld_x, arr[i].ld_out = r, c, c, c
    out = ctypes.c_size_t(0)
    _check(L.muon_ns_workspace_size(arr, len(shapes), _dtype_code(dtype), ctypes.byref(out)))
    return int(out.value)


def step_workspace_size(shapes) -> int:
    L = load()
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[int(r) for r, _ in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[int(c) for _, c in shapes])
    out = ctypes.c_size_t(0)
    _check(L.muon_step_workspace_size(rows, cols, n, ctypes.byref(out)))
    return int(out.value)


def step_selected_workspace_size(shapes, fraction: float) -> int:
    L = load()
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[int(r) for r, _ in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[int(c) for _, c in shapes])
    out = ctypes.c_size_t(0)
    _check(L.muon_step_selected_workspace_size(rows, cols, n, float(fraction), ctypes.byref(out)))
    return int(out.value)


def describe_plan(shapes, for_step=True, dtype=torch.bfloat16, steps=5, coeffs=QUINTIC) -> dict:
    L = load()
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[int(r) for r, _ in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[int(c) for _, c in shapes])
    buf = ctypes.create_string_buffer(1 << 20)
    _check(L.muon_describe_plan(rows, cols, n, int(bool(for_step)), _dtype_code(dtype), steps,
                                _coeffs(coeffs), buf, len(buf)))
    return json.loads(buf.value.decode())


def muon_ns_batched(xs, outs=None, steps: int = 5, coeffs=QUINTIC, eps: float = 1e-7,
                    workspace=None, stream=None):
    """outs[i] = NS_steps(xs[i] / (‖xs[i]‖_F + eps)) for every matrix, in one
    batched call.  All tensors: same device, dtype float32 or bfloat16, 2-D
    with contiguous rows.  Returns ``outs`` (allocated if None)."""
    L = load()
    xs = list(xs)
    if outs is None:
        outs = [torch.empty_like(x, memory_format=torch.contiguous_format) for x in xs]
    outs = list(outs)
    if len(outs) != len(xs):
        raise ValueError("xs and outs differ in length")
    if not xs:
        return outs
    dev, dt = _same_device_dtype(xs, outs)
    code = _dtype_code(dt)
    arr = _ns_descs(xs, outs)
    need = ctypes.c_size_t(0)
    _check(L.muon_ns_workspace_size(arr, len(xs), code, ctypes.byref(need)))
    ws, ws_bytes = _workspace(int(need.value), dev, workspace, stream)
    with torch.cuda.device(dev):
        _check(L.muon_ns_batched(arr, len(xs), int(steps), _coeffs(coeffs), code, float(eps),
                                 ctypes.c_void_p(ws.data_ptr() if ws is not None else 0),
                                 ws_bytes, _stream_handle(stream, dev)))
    return outs


def muon_ns_batched_noalloc(xs, outs, steps: int = 5, coeffs=QUINTIC, eps: float = 1e-7,
                            stream=None):
    """muon_ns_batched through the entry point that allocates nothing: the
    library's static per-device scratch serves as workspace, and the caller
    supplies the outputs (nothing is allocated here either).  Calls that may
    overlap on one device race for that scratch."""
    L = load()
    xs, outs = list(xs), list(outs)
    if len(outs) != len(xs):
        raise ValueError("xs and outs differ in length")
    if not xs:
        return outs
    dev, dt = _same_device_dtype(xs, outs)
    arr = _ns_descs(xs, outs)
    with torch.cuda.device(dev):
        _check(L.muon_ns_batched_noalloc(arr, len(xs), int(steps), _coeffs(coeffs), _dtype_code(dt),
                                         float(eps), _stream_handle(stream, dev)))
    return outs


def muon_step(params, grads, momenta, beta: float = 0.95, lr: float = 0.02, steps: int = 5,
              coeffs=QUINTIC, eps: float = 1e-7, workspace=None, stream=None,
              nesterov: bool = False, weight_decay: float = 0.0, overlap: bool = False,
              max_workspace_bytes: int = 0, scale_exp=None):
    """One in-place Muon step over lists of weights (bf16 or fp32), gradients
    (fp32 or bf16, one dtype per call) and fp32 momenta (all contiguous, same
    device).  nesterov / weight_decay / overlap / max_workspace_bytes /
    scale_exp select the muon_step_ex options (see muon_step_opts_t); with
    their defaults and fp32 gradients the plain muon_step entry point runs.
    With a budget the cached workspace is at most max_workspace_bytes.
    scale_exp: None or a contiguous int32 tensor of len(params) entries on the
    params' device (see scale_exp_buffer), read and rewritten by the call."""
    L = load()
    params, grads, momenta = list(params), list(grads), list(momenta)
    n = len(params)
    if not (len(grads) == len(momenta) == n):
        raise ValueError("params, grads and momenta differ in length")
    if n == 0:
        return
    dev = params[0].device
    pdt = params[0].dtype
    gdt = grads[0].dtype
    if gdt not in (torch.float32, torch.bfloat16):
        raise TypeError("grads must be float32 or bfloat16")
    for p, g, m in zip(params, grads, momenta):
        if p.device != dev or g.device != dev or m.device != dev or dev.type != "cuda":
            raise ValueError("all tensors must be on one CUDA/HIP device")
        if p.dtype != pdt:
            raise TypeError("all params must share one dtype")
        if g.dtype != gdt:
            raise TypeError("all grads must share one dtype")
        if m.dtype != torch.float32:
            raise TypeError("momenta must be float32")
        if p.dim() != 2 or tuple(p.shape) != tuple(g.shape) or tuple(p.shape) != tuple(m.shape):
            raise ValueError("param, grad and momentum shapes differ (or not 2-D)")
        if not (p.is_contiguous() and g.is_contiguous() and m.is_contiguous()):
            raise ValueError("params, grads and momenta must be contiguous")
    vp = ctypes.c_void_p
    P = (vp * n)(*[p.data_ptr() for p in params])
    G = (vp * n)(*[g.data_ptr() for g in grads])
    M = (vp * n)(*[m.data_ptr() for m in momenta])
    rows = (ctypes.c_int64 * n)(*[int(p.shape[0]) for p in params])
    cols = (ctypes.c_int64 * n)(*[int(p.shape[1]) for p in params])
    if scale_exp is not None:
        if (scale_exp.dtype != torch.int32 or scale_exp.device != dev or not scale_exp.is_contiguous()
                or scale_exp.numel() != n):
            raise ValueError("scale_exp must be a contiguous int32 tensor of len(params) entries "
                             "on the params' device")
    need = ctypes.c_size_t(0)
    _check(L.muon_step_workspace_size(rows, cols, n, ctypes.byref(need)))
    nbytes = int(need.value)
    if max_workspace_bytes:
        nbytes = min(nbytes, int(max_workspace_bytes))
    ws, ws_bytes = _workspace(nbytes, dev, workspace, stream)
    plain = ((not nesterov) and float(weight_decay) == 0.0 and gdt == torch.float32 and not overlap
             and not max_workspace_bytes and scale_exp is None)
    with torch.cuda.device(dev):
        wsp = ctypes.c_void_p(ws.data_ptr() if ws is not None else 0)
        if plain:
            _check(L.muon_step(P, G, M, rows, cols, n, _dtype_code(pdt), float(beta), float(lr),
                               int(steps), _coeffs(coeffs), float(eps), wsp, ws_bytes,
                               _stream_handle(stream, dev)))
        else:
            opts = MuonStepOpts(int(bool(nesterov)), float(weight_decay), _dtype_code(gdt),
                                int(bool(overlap)), int(max_workspace_bytes),
                                scale_exp.data_ptr() if scale_exp is not None else None)
            _check(L.muon_step_ex(P, G, M, rows, cols, n, _dtype_code(pdt), float(beta),
                                  float(lr), int(steps), _coeffs(coeffs), float(eps),
                                  ctypes.byref(opts), wsp, ws_bytes, _stream_handle(stream, dev)))


def muon_step_selected(params, grads, momenta, fraction: float, beta: float = 0.95, lr: float = 0.02,
                       steps: int = 5, coeffs=QUINTIC, eps: float = 1e-7, workspace=None, stream=None):
    """One in-place row/column-selected Muon step with error feedback (the
    muon_step_selected entry point): per matrix only the ⌈fraction·m⌉
    highest-norm rows of B = M + g along the short side are orthogonalised
    and applied; the buffer keeps B elsewhere and β·B on the selection.
    params bf16 or fp32, grads and momenta fp32, all contiguous on one device."""
    L = load()
    params, grads, momenta = list(params), list(grads), list(momenta)
    n = len(params)
    if not (len(grads) == len(momenta) == n):
        raise ValueError("params, grads and momenta differ in length")
    if n == 0:
        return
    dev = params[0].device
    pdt = params[0].dtype
    for p, g, m in zip(params, grads, momenta):
        if p.device != dev or g.device != dev or m.device != dev or dev.type != "cuda":
            raise ValueError("all tensors must be on one CUDA/HIP device")
        if p.dtype != pdt:
            raise TypeError("all params must share one dtype")
        if g.dtype != torch.float32 or m.dtype != torch.float32:
            raise TypeError("grads and momenta must be float32")
        if p.dim() != 2 or tuple(p.shape) != tuple(g.shape) or tuple(p.shape) != tuple(m.shape):
            raise ValueError("param, grad and momentum shapes differ (or not 2-D)")
        if not (p.is_contiguous() and g.is_contiguous() and m.is_contiguous()):
            raise ValueError("params, grads and momenta must be contiguous")
    vp = ctypes.c_void_p
    P = (vp * n)(*[p.data_ptr() for p in params])
    G = (vp * n)(*[g.data_ptr() for g in grads])
    M = (vp * n)(*[m.data_ptr() for m in momenta])
    rows = (ctypes.c_int64 * n)(*[int(p.shape[0]) for p in params])
    cols = (ctypes.c_int64 * n)(*[int(p.shape[1]) for p in params])
    need = ctypes.c_size_t(0)
    _check(L.muon_step_selected_workspace_size(rows, cols, n, float(fraction), ctypes.byref(need)))
    ws, ws_bytes = _workspace(int(need.value), dev, workspace, stream)
    with torch.cuda.device(dev):
        wsp = ctypes.c_void_p(ws.data_ptr() if ws is not None else 0)
        _check(L.muon_step_selected(P, G, M, rows, cols, n, _dtype_code(pdt), float(beta), float(lr),
                                    int(steps), _coeffs(coeffs), float(eps), float(fraction), wsp,
                                    ws_bytes, _stream_handle(stream, dev)))


def set_tile_table(entries):
    """Install the planner's tuning table: an iterable of dicts with keys m,
    op ("f16" or "f32"), count_class (floor(log2(matrices in the group))) and
    optionally n (the group's largest n; 0 or absent: any), tile,
    xcd_window and band (0 or absent: built-in).  An empty iterable clears
    it."""
    entries = list(entries)
    arr = (MuonTileEntry * max(len(entries), 1))()
    for i, e in enumerate(entries):
        op = e["op"]
        arr[i].m = int(e["m"])
        arr[i].n = int(e.get("n", 0))
        arr[i].op = {"f16": 0, "f32": 1}[op] if isinstance(op, str) else int(op)
        arr[i].count_class = int(e["count_class"])
        arr[i].tile = int(e.get("tile", 0))
        arr[i].xcd_window = int(e.get("xcd_window", 0))
        arr[i].band = int(e.get("band", 0))
    _check(load().muon_set_tile_table(arr, len(entries)))


def profile_enable(on: bool = True):
    _check(load().muon_profile_enable(int(bool(on))))


def profile_read(kind) -> dict:
    """Totals of the launches recorded for one kind since the last read:
    {"ms": total kernel ms, "launches": n, "work": algorithmic flops or bytes}."""
    k = PROFILE_KINDS[kind] if isinstance(kind, str) else int(kind)
    ms, n, w = ctypes.c_double(0), ctypes.c_int64(0), ctypes.c_double(0)
    _check(load().muon_profile_read(k, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(w)))
    return {"ms": ms.value, "launches": n.value, "work": w.value}


from .optim import Muon  # noqa: E402  (torch.optim front end)

__all__.append("Muon")
