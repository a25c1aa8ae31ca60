"""ctypes binding of libmuon_rocm.so (include/muon_rocm.h).

Argument marshalling only: every step of the optimizer runs in the library's HIP
kernels. torch tensors provide device memory and the current HIP stream. If the
library is not built, or no GPU is present, calls raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

from .build import LIB_PATH

MUON_OK = 0
MUON_ERR_INVALID_ARG = -1
MUON_ERR_WORKSPACE = -2
MUON_ERR_ALIGN = -3
MUON_ERR_ALIAS = -4
MUON_ERR_HIP = -5
MUON_ERR_TOO_LARGE = -6

# update-scale rules (include/muon_rocm.h)
SCALE_MAX_DIM = 0   # 0.2 sqrt(max(A, B)), Eq. 4 / Eq. 7
SCALE_HIDDEN = 1    # 0.2 sqrt(H), Eq. 5
SCALE_RMS = 2       # 0.2 / RMS(O), Eq. 6

KCLASS_NAMES = ("cast", "frob", "gram", "poly", "apply", "apply_final", "rownorm_rows",
                "colnorm_partial", "colnorm_finalize", "colnorm_apply", "rms_finalize",
                "scaled_update", "adamw", "spec_gram", "spec_house", "spec_pass", "spec_reduce",
                "spec_bisect", "spec_entropy")

EXPORTED = ("muon_abi_version", "muon_status_str", "muon_last_error", "muon_default_hparams",
            "muon_workspace_bytes", "ns5_plan", "muon_step", "ns5_batched", "rownorm_update",
            "rownorm_update_noalloc",
            "adamw_default_hparams", "adamw_step", "svd_entropy_workspace_bytes", "svd_entropy",
            "rownorm_shard_workspace_bytes", "rownorm_shard_colsq", "rownorm_shard_apply",
            "muon_ceiling_copy", "muon_ceiling_mfma", "muon_timing_enable", "muon_timing_read")


class MuonHParams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float), ("weight_decay", ctypes.c_float), ("mu", ctypes.c_float),
        ("ns_a", ctypes.c_float), ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float),
        ("rms_scale", ctypes.c_float), ("gamma", ctypes.c_float), ("eps", ctypes.c_float),
        ("ns_steps", ctypes.c_int32), ("period_k", ctypes.c_int32),
        ("scale_mode", ctypes.c_int32), ("hidden", ctypes.c_int32),
    ]


class MuonMatrix(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("w", ctypes.c_void_p),
                ("m", ctypes.c_void_p), ("g", ctypes.c_void_p)]


class AdamWHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


class AdamWParam(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("w", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("g", ctypes.c_void_p)]


class MuonShard(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("full_rows", ctypes.c_int64),
                ("w", ctypes.c_void_p), ("m", ctypes.c_void_p), ("g", ctypes.c_void_p)]


class MuonError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = f"{where}: status {status} ({status_str(status)})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


_lib: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmuon_rocm.so (built in-tree by build.build()); raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    # MUON_ROCM_LIBRARY selects another build of the same library (the host-sanitized
    # one in the CPU sanitizer run)
    p = path or os.environ.get("MUON_ROCM_LIBRARY") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run matrix_orthogonalising_optimizer_02_amd.build.build()")
    lib = ctypes.CDLL(p)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.muon_abi_version.restype = ctypes.c_int
    lib.muon_status_str.restype = ctypes.c_char_p
    lib.muon_status_str.argtypes = [ctypes.c_int]
    lib.muon_last_error.restype = ctypes.c_char_p
    lib.muon_default_hparams.argtypes = [ctypes.POINTER(MuonHParams)]
    lib.muon_default_hparams.restype = None
    lib.muon_workspace_bytes.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64), i32,
                                         ctypes.POINTER(ctypes.c_size_t)]
    lib.ns5_plan.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64), i32,
                             ctypes.POINTER(ctypes.c_int32), i32, ctypes.POINTER(ctypes.c_int32)]
    lib.muon_step.argtypes = [ctypes.POINTER(MuonMatrix), i32, ctypes.POINTER(MuonHParams), i64, vp, sz, vp, vp]
    lib.ns5_batched.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_int64),
                                ctypes.POINTER(ctypes.c_int64), i32, ctypes.POINTER(MuonHParams), vp, sz, vp]
    lib.rownorm_update.argtypes = [ctypes.POINTER(MuonMatrix), i32, ctypes.POINTER(MuonHParams), vp, sz, vp, vp]
    lib.rownorm_update_noalloc.argtypes = [ctypes.POINTER(MuonMatrix), i32, ctypes.POINTER(MuonHParams), vp, vp]
    lib.adamw_default_hparams.argtypes = [ctypes.POINTER(AdamWHParams)]
    lib.adamw_default_hparams.restype = None
    lib.adamw_step.argtypes = [ctypes.POINTER(AdamWParam), i32, ctypes.POINTER(AdamWHParams), i64, vp]
    lib.svd_entropy_workspace_bytes.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                                i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.svd_entropy.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                i32, vp, sz, vp, vp, vp]
    lib.rownorm_shard_workspace_bytes.argtypes = [ctypes.POINTER(MuonShard), i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.rownorm_shard_colsq.argtypes = [ctypes.POINTER(MuonShard), i32, ctypes.POINTER(MuonHParams),
                                        ctypes.POINTER(vp), vp, sz, vp]
    lib.rownorm_shard_apply.argtypes = [ctypes.POINTER(MuonShard), i32, ctypes.POINTER(MuonHParams),
                                        ctypes.POINTER(vp), vp, sz, vp]
    lib.muon_ceiling_copy.argtypes = [vp, vp, i64, vp]
    lib.muon_ceiling_mfma.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_double), vp]
    lib.muon_timing_enable.argtypes = [ctypes.c_int]
    lib.muon_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    for name in ("muon_step", "ns5_batched", "rownorm_update", "rownorm_update_noalloc", "muon_workspace_bytes",
                 "ns5_plan", "adamw_step", "svd_entropy_workspace_bytes", "svd_entropy", "rownorm_shard_workspace_bytes",
                 "rownorm_shard_colsq", "rownorm_shard_apply", "muon_ceiling_copy", "muon_ceiling_mfma",
                 "muon_timing_enable", "muon_timing_read"):
        getattr(lib, name).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().muon_status_str(status).decode()


def _check(rc: int, where: str):
    if rc != MUON_OK:
        detail = load_library().muon_last_error().decode()
        raise MuonError(rc, where, detail)


def default_hparams(**overrides) -> MuonHParams:
    hp = MuonHParams()
    load_library().muon_default_hparams(ctypes.byref(hp))
    for k, v in overrides.items():
        if not hasattr(hp, k):
            raise KeyError(k)
        setattr(hp, k, v)
    return hp


def workspace_bytes(shapes: Sequence[Sequence[int]]) -> int:
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[int(s[0]) for s in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[int(s[1]) for s in shapes])
    out = ctypes.c_size_t(0)
    _check(load_library().muon_workspace_bytes(rows, cols, n, ctypes.byref(out)), "muon_workspace_bytes")
    return int(out.value)


PLAN_RECORD_INTS = 85
PLAN_STAGES = ("gram", "poly", "apply", "apply_final")


def ns5_plan(shapes: Sequence[Sequence[int]]):
    """The Newton-Schulz GEMM plan the library uses for these shapes (host only): one
    dict per group with the matrices' indices and, per stage, (tile width, {XCD: (split
    tiles, chunks)}) for the XCDs that split. Split tiles > 0: that many tiles of the
    XCD's last round run as K chunks (tail split); < 0: its first -h tiles do (head
    split of a one-round stage with mixed K)."""
    lib = load_library()
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[int(s[0]) for s in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[int(s[1]) for s in shapes])
    ng = ctypes.c_int32(0)
    _check(lib.ns5_plan(rows, cols, n, None, 0, ctypes.byref(ng)), "ns5_plan")
    cap = max(ng.value, 1) * PLAN_RECORD_INTS
    out = (ctypes.c_int32 * cap)()
    _check(lib.ns5_plan(rows, cols, n, out, cap, ctypes.byref(ng)), "ns5_plan")
    groups = []
    for g in range(ng.value):
        r = out[g * PLAN_RECORD_INTS:(g + 1) * PLAN_RECORD_INTS]
        rec = {"indices": [int(v) for v in r[1:1 + r[0]]]}
        for st, name in enumerate(PLAN_STAGES):
            q = r[17 + 17 * st:34 + 17 * st]
            rec[name] = (int(q[0]), {x: (int(q[1 + 2 * x]), int(q[2 + 2 * x])) for x in range(8) if q[1 + 2 * x] != 0})
        groups.append(rec)
    return groups


# ------------------------------------------------------------ tensor helpers ----

def _torch():
    import torch
    return torch


def _check_tensor(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32 or t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D float32 tensor")
    if t.numel() and t.device.type != "cuda":
        raise ValueError(f"{name} must live on a GPU")


def _stream_handle(stream, device=None):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(int(getattr(stream, "cuda_stream", stream)))


def make_workspace(shapes, device="cuda"):
    """A uint8 device buffer large enough for every entry point on `shapes`."""
    torch = _torch()
    return torch.empty(max(workspace_bytes(shapes), 1), dtype=torch.uint8, device=device)


def _torch_stream(stream, device):
    """The torch stream object for `stream` (None: the device's current stream)."""
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)), device=device)


def _scratch(nbytes, device, stream):
    """A device buffer for one library call, allocated on the stream the call enqueues on.

    torch's caching allocator keeps a freed block with the stream it was allocated on
    and hands it out again only to allocations on that stream, which run after the
    call's kernels in stream order. A buffer allocated on another stream could be
    reused there while the call's kernels still write it.
    """
    torch = _torch()
    with torch.cuda.stream(_torch_stream(stream, device)):
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _ws(workspace, shapes, device, stream):
    """(pointer, size, owner) of the call's workspace; `owner` must stay referenced until
    the library call has returned."""
    if workspace is None:
        workspace = _scratch(workspace_bytes(shapes), device, stream)
    return ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()), workspace


def _matrices(weights, momenta, grads):
    if not (len(weights) == len(momenta) == len(grads)):
        raise ValueError("weights, momenta and grads must have the same length")
    arr = (MuonMatrix * max(len(weights), 1))()
    for i, (w, m, g) in enumerate(zip(weights, momenta, grads)):
        for t, nm in ((w, "weight"), (m, "momentum"), (g, "grad")):
            _check_tensor(t, f"{nm}[{i}]")
        if not (w.shape == m.shape == g.shape):
            raise ValueError(f"shape mismatch at index {i}")
        arr[i] = MuonMatrix(w.shape[0], w.shape[1], w.data_ptr() or None, m.data_ptr() or None,
                            g.data_ptr() or None)
    return arr


def _monitor_ptr(update_rms, count):
    """Device pointer of an optional float32 [count] tensor for the update-RMS monitor."""
    if update_rms is None:
        return ctypes.c_void_p(None)
    torch = _torch()
    if not isinstance(update_rms, torch.Tensor) or update_rms.dtype != torch.float32 \
            or update_rms.dim() != 1 or not update_rms.is_contiguous() or update_rms.numel() != count:
        raise ValueError("update_rms must be a contiguous float32 tensor with one entry per matrix")
    if count and update_rms.device.type != "cuda":
        raise ValueError("update_rms must live on a GPU")
    return ctypes.c_void_p(update_rms.data_ptr() or None)


def muon_step(weights, momenta, grads, step: int, hp: Optional[MuonHParams] = None,
              workspace=None, stream=None, update_rms=None):
    """One Periodic Row-wise Muon step (refresh iff step % period_k == 0), in place.

    update_rms: optional float32 device tensor [len(weights)] that receives each
    matrix's update RMS (RMS of the scaled direction, before lr and weight decay).
    """
    hp = hp or default_hparams()
    arr = _matrices(weights, momenta, grads)
    dev = weights[0].device if weights else None
    ws, wsb, _owner = _ws(workspace, [tuple(w.shape) for w in weights], dev, stream)
    rc = load_library().muon_step(arr, len(weights), ctypes.byref(hp), int(step), ws, wsb,
                                  _monitor_ptr(update_rms, len(weights)), _stream_handle(stream, dev))
    _check(rc, "muon_step")


def rownorm_update(weights, momenta, grads, hp: Optional[MuonHParams] = None, workspace=None,
                   stream=None, update_rms=None):
    """The Periodic variant's RowNorm step, in place (update_rms as for muon_step)."""
    hp = hp or default_hparams()
    arr = _matrices(weights, momenta, grads)
    dev = weights[0].device if weights else None
    ws, wsb, _owner = _ws(workspace, [tuple(w.shape) for w in weights], dev, stream)
    rc = load_library().rownorm_update(arr, len(weights), ctypes.byref(hp), ws, wsb,
                                       _monitor_ptr(update_rms, len(weights)), _stream_handle(stream, dev))
    _check(rc, "rownorm_update")


def rownorm_update_noalloc(weights, momenta, grads, hp: Optional[MuonHParams] = None, stream=None,
                           update_rms=None):
    """rownorm_update on the library's fixed device scratch: allocates nothing (for graph
    capture and serving loops). Calls that overlap in time on one GPU race."""
    hp = hp or default_hparams()
    arr = _matrices(weights, momenta, grads)
    dev = weights[0].device if weights else None
    rc = load_library().rownorm_update_noalloc(arr, len(weights), ctypes.byref(hp),
                                               _monitor_ptr(update_rms, len(weights)), _stream_handle(stream, dev))
    _check(rc, "rownorm_update_noalloc")


def ns5_batched(inputs, outputs=None, hp: Optional[MuonHParams] = None, workspace=None, stream=None):
    """outputs[i] = NS5(inputs[i]); returns the outputs (new tensors when not given)."""
    torch = _torch()
    hp = hp or default_hparams()
    if outputs is None:
        outputs = [torch.empty_like(x) for x in inputs]
    if len(outputs) != len(inputs):
        raise ValueError("inputs and outputs must have the same length")
    n = len(inputs)
    ins = (ctypes.c_void_p * max(n, 1))()
    outs = (ctypes.c_void_p * max(n, 1))()
    rows = (ctypes.c_int64 * max(n, 1))()
    cols = (ctypes.c_int64 * max(n, 1))()
    for i, (x, o) in enumerate(zip(inputs, outputs)):
        _check_tensor(x, f"inputs[{i}]")
        _check_tensor(o, f"outputs[{i}]")
        if x.shape != o.shape:
            raise ValueError(f"shape mismatch at index {i}")
        ins[i] = x.data_ptr() or None
        outs[i] = o.data_ptr() or None
        rows[i], cols[i] = x.shape
    dev = inputs[0].device if inputs else None
    ws, wsb, _owner = _ws(workspace, [tuple(x.shape) for x in inputs], dev, stream)
    rc = load_library().ns5_batched(ins, outs, rows, cols, n, ctypes.byref(hp), ws, wsb,
                                    _stream_handle(stream, dev))
    _check(rc, "ns5_batched")
    return outputs


def adamw_default_hparams(**overrides) -> AdamWHParams:
    hp = AdamWHParams()
    load_library().adamw_default_hparams(ctypes.byref(hp))
    for k, v in overrides.items():
        if not hasattr(hp, k):
            raise KeyError(k)
        setattr(hp, k, v)
    return hp


def _check_flat(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor")
    if t.numel() and t.device.type != "cuda":
        raise ValueError(f"{name} must live on a GPU")


class AdamWGroup:
    """Tensors for repeated AdamW steps, with the C descriptor array built once.

    The gradient tensors given here are read at every step (write each step's gradients
    into them in place), unless step() is passed a new list.
    """

    def __init__(self, params, grads, exp_avgs, exp_avg_sqs, hp: Optional[AdamWHParams] = None):
        n = len(params)
        if not (n == len(grads) == len(exp_avgs) == len(exp_avg_sqs)):
            raise ValueError("params, grads and moment lists must have the same length")
        self.hp = hp or adamw_default_hparams()
        self.tensors = (list(params), list(grads), list(exp_avgs), list(exp_avg_sqs))
        self.arr = (AdamWParam * max(n, 1))()
        for i, (w, g, m, v) in enumerate(zip(params, grads, exp_avgs, exp_avg_sqs)):
            for t, nm in ((w, "param"), (g, "grad"), (m, "exp_avg"), (v, "exp_avg_sq")):
                _check_flat(t, f"{nm}[{i}]")
            if not (w.shape == g.shape == m.shape == v.shape):
                raise ValueError(f"shape mismatch at index {i}")
            self.arr[i] = AdamWParam(w.numel(), w.data_ptr() or None, m.data_ptr() or None,
                                     v.data_ptr() or None, g.data_ptr() or None)
        self.n = n
        self.device = params[0].device if params else None

    def set_grads(self, grads):
        if len(grads) != self.n:
            raise ValueError("one gradient per parameter")
        for i, (g, w) in enumerate(zip(grads, self.tensors[0])):
            _check_flat(g, f"grad[{i}]")
            if g.shape != w.shape:
                raise ValueError(f"shape mismatch at index {i}")
            self.arr[i].g = g.data_ptr() or None
        self.tensors = (self.tensors[0], list(grads), self.tensors[2], self.tensors[3])

    def step(self, step: int, stream=None, grads=None):
        if grads is not None:
            self.set_grads(grads)
        rc = load_library().adamw_step(self.arr, self.n, ctypes.byref(self.hp), int(step),
                                       _stream_handle(stream, self.device))
        _check(rc, "adamw_step")


def adamw_step(params, grads, exp_avgs, exp_avg_sqs, step: int, hp: Optional[AdamWHParams] = None,
               stream=None):
    """One AdamW step (0-based `step`) over tensors of any shape, in place."""
    AdamWGroup(params, grads, exp_avgs, exp_avg_sqs, hp).step(step, stream)


# ------------------------------------------------ row-sharded RowNorm share ----

def _shards(weights, momenta, grads, full_rows):
    n = len(weights)
    if not (n == len(momenta) == len(full_rows)) or (grads is not None and len(grads) != n):
        raise ValueError("weights, momenta, grads and full_rows must have the same length")
    arr = (MuonShard * max(n, 1))()
    for i in range(n):
        w, m = weights[i], momenta[i]
        g = grads[i] if grads is not None else None
        for t, nm in ((w, "weight"), (m, "momentum")) + (((g, "grad"),) if g is not None else ()):
            _check_tensor(t, f"{nm}[{i}]")
        if w.shape != m.shape or (g is not None and g.shape != w.shape):
            raise ValueError(f"shape mismatch at index {i}")
        arr[i] = MuonShard(w.shape[0], w.shape[1], int(full_rows[i]), w.data_ptr() or None,
                           m.data_ptr() or None, (g.data_ptr() or None) if g is not None else None)
    return arr


def rownorm_shard_workspace_bytes(shapes, full_rows) -> int:
    arr = (MuonShard * max(len(shapes), 1))()
    for i, (s, a) in enumerate(zip(shapes, full_rows)):
        arr[i] = MuonShard(int(s[0]), int(s[1]), int(a), None, None, None)
    out = ctypes.c_size_t(0)
    _check(load_library().rownorm_shard_workspace_bytes(arr, len(shapes), ctypes.byref(out)),
           "rownorm_shard_workspace_bytes")
    return int(out.value)


def _shard_ws(workspace, weights, full_rows, dev, stream):
    """As _ws, for the shard calls."""
    if workspace is None:
        nb = rownorm_shard_workspace_bytes([tuple(w.shape) for w in weights], full_rows)
        workspace = _scratch(nb, dev, stream)
    return ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()), workspace


def _sum_ptrs(tensors, weights, name):
    torch = _torch()
    if len(tensors) != len(weights):
        raise ValueError(f"{name} needs one column-sum tensor per block")
    ptrs = (ctypes.c_void_p * max(len(weights), 1))()
    for i, (t, w) in enumerate(zip(tensors, weights)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 1 \
                or not t.is_contiguous() or t.numel() != w.shape[1]:
            raise ValueError(f"{name}[{i}] must be a contiguous float32 tensor of {w.shape[1]} entries")
        ptrs[i] = t.data_ptr() or None
    return ptrs


def rownorm_shard_colsq(weights, momenta, grads, full_rows, colsq=None, hp: Optional[MuonHParams] = None,
                        workspace=None, stream=None):
    """Step 1 of a tall matrix's row-sharded RowNorm step on this GPU's blocks: momentum,
    and the block's column sums of M'^2 (returned; reduce them across the GPUs)."""
    torch = _torch()
    hp = hp or default_hparams()
    dev = weights[0].device if weights else None
    if colsq is None:
        colsq = [torch.empty(w.shape[1], dtype=torch.float32, device=dev) for w in weights]
    arr = _shards(weights, momenta, grads, full_rows)
    ws, wsb, _owner = _shard_ws(workspace, weights, full_rows, dev, stream)
    rc = load_library().rownorm_shard_colsq(arr, len(weights), ctypes.byref(hp), _sum_ptrs(colsq, weights, "colsq"),
                                            ws, wsb, _stream_handle(stream, dev))
    _check(rc, "rownorm_shard_colsq")
    return colsq


def rownorm_shard_apply(weights, momenta, full_rows, colsq_total, hp: Optional[MuonHParams] = None,
                        workspace=None, stream=None):
    """Step 3: the column-normalised update of this GPU's blocks from the reduced sums."""
    hp = hp or default_hparams()
    dev = weights[0].device if weights else None
    arr = _shards(weights, momenta, None, full_rows)
    ws, wsb, _owner = _shard_ws(workspace, weights, full_rows, dev, stream)
    rc = load_library().rownorm_shard_apply(arr, len(weights), ctypes.byref(hp),
                                            _sum_ptrs(colsq_total, weights, "colsq_total"), ws, wsb,
                                            _stream_handle(stream, dev))
    _check(rc, "rownorm_shard_apply")


# ------------------------------------------------------- spectrum diagnostic ----

def _shape_arrays(shapes):
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[int(s[0]) for s in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[int(s[1]) for s in shapes])
    return rows, cols


def svd_entropy_workspace_bytes(shapes: Sequence[Sequence[int]]) -> int:
    rows, cols = _shape_arrays(shapes)
    out = ctypes.c_size_t(0)
    _check(load_library().svd_entropy_workspace_bytes(rows, cols, len(shapes), ctypes.byref(out)),
           "svd_entropy_workspace_bytes")
    return int(out.value)


def make_svd_entropy_workspace(shapes, device="cuda"):
    torch = _torch()
    return torch.empty(max(svd_entropy_workspace_bytes(shapes), 1), dtype=torch.uint8, device=device)


def svd_entropy(weights, entropy=None, sigma_sq=None, workspace=None, stream=None):
    """SVD entropy of each 2-D fp32 device matrix ("Muon is Scalable", Sec. 3.4).

    Returns the float64 device tensor `entropy` [len(weights)] (new when not given).
    sigma_sq: optional float64 device tensor of sum(min(A, B)) entries that receives
    every matrix's squared singular values, descending, one matrix after another.
    """
    torch = _torch()
    n = len(weights)
    dev = weights[0].device if weights else None
    for i, w in enumerate(weights):
        _check_tensor(w, f"weights[{i}]")
    shapes = [tuple(w.shape) for w in weights]
    if entropy is None:
        entropy = torch.full((n,), float("nan"), dtype=torch.float64, device=dev)
    for t, nm, size in ((entropy, "entropy", n), (sigma_sq, "sigma_sq", sum(min(s) for s in shapes))):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float64 or t.dim() != 1 \
                or not t.is_contiguous() or t.numel() != size:
            raise ValueError(f"{nm} must be a contiguous float64 tensor of {size} entries")
        if size and t.device.type != "cuda":
            raise ValueError(f"{nm} must live on a GPU")
    ptrs = (ctypes.c_void_p * max(n, 1))(*[w.data_ptr() or None for w in weights])
    rows, cols = _shape_arrays(shapes)
    if workspace is None:
        workspace = _scratch(svd_entropy_workspace_bytes(shapes), dev, stream)
    rc = load_library().svd_entropy(ptrs, rows, cols, n, ctypes.c_void_p(workspace.data_ptr()),
                                    ctypes.c_size_t(workspace.numel()),
                                    ctypes.c_void_p(entropy.data_ptr() or None),
                                    ctypes.c_void_p(sigma_sq.data_ptr() if sigma_sq is not None else None),
                                    _stream_handle(stream, dev))
    _check(rc, "svd_entropy")
    return entropy


def ceiling_copy(src, dst, stream=None):
    """dst <- src through the library's streaming copy kernel (the HBM yardstick)."""
    _check_flat(src, "src")
    _check_flat(dst, "dst")
    if src.numel() != dst.numel():
        raise ValueError("src and dst must have the same number of elements")
    rc = load_library().muon_ceiling_copy(ctypes.c_void_p(src.data_ptr() or None),
                                          ctypes.c_void_p(dst.data_ptr() or None), src.numel(),
                                          _stream_handle(stream, src.device))
    _check(rc, "muon_ceiling_copy")


def ceiling_mfma(out, blocks: int, iters: int, stream=None) -> float:
    """The register-only bf16 MFMA loop (the MFMA yardstick) over `blocks` blocks; `out`
    is a float32 device tensor of 4 * blocks checksums. Returns the dense flop count."""
    _check_flat(out, "out")
    if out.numel() < 4 * blocks:
        raise ValueError("out needs 4 entries per block")
    flops = ctypes.c_double(0.0)
    rc = load_library().muon_ceiling_mfma(ctypes.c_void_p(out.data_ptr() or None), int(blocks), int(iters),
                                          ctypes.byref(flops), _stream_handle(stream, out.device))
    _check(rc, "muon_ceiling_mfma")
    return flops.value


def timing_enable(enable: bool = True):
    _check(load_library().muon_timing_enable(1 if enable else 0), "muon_timing_enable")


def timing_read():
    """{kernel class: (total ms, launches)} since the last read; waits for the events."""
    ms = (ctypes.c_double * len(KCLASS_NAMES))()
    cnt = (ctypes.c_int64 * len(KCLASS_NAMES))()
    _check(load_library().muon_timing_read(ms, cnt), "muon_timing_read")
    return {name: (ms[i], int(cnt[i])) for i, name in enumerate(KCLASS_NAMES)}


class MuonOptimizer:
    """Periodic Row-wise Muon over a list of 2-D fp32 CUDA parameters.

    Holds one momentum buffer per parameter (zeros at step 0), the workspace and the
    step counter; step(grads) advances every parameter by one optimizer step.
    """

    def __init__(self, params, hp: Optional[MuonHParams] = None):
        torch = _torch()
        self.params = list(params)
        self.hp = hp or default_hparams()
        self.momenta = [torch.zeros_like(p) for p in self.params]
        self.workspace = make_workspace([tuple(p.shape) for p in self.params],
                                        self.params[0].device if self.params else "cuda")
        self.step_count = 0

    def step(self, grads, stream=None, update_rms=None):
        muon_step(self.params, self.momenta, list(grads), self.step_count, self.hp,
                  self.workspace, stream, update_rms)
        self.step_count += 1

    def state_dict(self):
        return {"step": self.step_count, "momenta": [m.clone() for m in self.momenta]}

    def load_state_dict(self, state):
        self.step_count = int(state["step"])
        for dst, src in zip(self.momenta, state["momenta"]):
            dst.copy_(src)

