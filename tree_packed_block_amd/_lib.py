"""ctypes binding of ``liboctopus_dag.so`` (argument marshalling only).

Every step of the path runs inside the library: planning on the host in C++, all
attention and decode arithmetic in HIP kernels.  PyTorch only supplies device memory
and the current stream.  If the library is missing the calls raise; there is no
fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboctopus_dag.so")

OK, EINVAL, ECYCLE, EUNSUPPORTED, ENOMEM, EWORKSPACE, EHIP, ESTATE = 0, -1, -2, -3, -4, -5, -6, -7
_NAMES = {EINVAL: "EINVAL", ECYCLE: "ECYCLE", EUNSUPPORTED: "EUNSUPPORTED",
          ENOMEM: "ENOMEM", EWORKSPACE: "EWORKSPACE", EHIP: "EHIP", ESTATE: "ESTATE"}
BF16, FP32 = 0, 1
DECODE_SCRATCH_BYTES = 48 << 20  # OCTOPUS_DECODE_SCRATCH_BYTES

# Every symbol include/octopus_dag.h declares.
EXPORTS = [
    "octopus_dag_plan", "octopus_plan_positions", "octopus_plan_stats_get",
    "octopus_plan_device_bytes", "octopus_plan_upload", "octopus_plan_export_mask",
    "octopus_plan_export_tiles", "octopus_plan_destroy", "octopus_fwd_workspace_bytes", "octopus_dag_attn_fwd",
    "octopus_bwd_workspace_bytes", "octopus_dag_attn_bwd", "octopus_dag_attn_bwd_preprocess",
    "octopus_dag_attn_bwd_dkdv", "octopus_dag_attn_bwd_dq", "octopus_decode_segments",
    "octopus_decode_workspace_bytes", "octopus_paged_mount_decode",
    "octopus_paged_mount_decode_noalloc", "octopus_extend_segments",
    "octopus_paged_mount_extend", "octopus_dag_positions", "octopus_rope",
    "octopus_rope_workspace_bytes", "octopus_dag_attn_fwd_rope", "octopus_dag_attn_bwd_rope",
    "octopus_gdn_workspace_bytes", "octopus_gated_delta_scan",
    "octopus_gdn_bwd_workspace_bytes", "octopus_gated_delta_scan_bwd",
    "octopus_gated_delta_scan_save", "octopus_gated_delta_scan_bwd_saved", "octopus_last_error",
    "octopus_version",
]


class OctopusError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code
        self.name = _NAMES.get(code, str(code))


class Stats(ctypes.Structure):
    _fields_ = [("nnz", ctypes.c_int64), ("n_pairs", ctypes.c_int64),
                ("n_partial", ctypes.c_int64), ("total_tokens", ctypes.c_int32),
                ("q_tile", ctypes.c_int32), ("kv_tile", ctypes.c_int32),
                ("n_q_tiles", ctypes.c_int32), ("n_kv_tiles", ctypes.c_int32),
                ("max_q_list", ctypes.c_int32), ("max_kv_list", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_lib = None
_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p


def lib():
    """Load the library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    L.octopus_dag_plan.argtypes = [_vp, ctypes.c_int32, _vp, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.POINTER(_vp)]
    L.octopus_plan_positions.argtypes = [_vp, _i32p]
    L.octopus_plan_stats_get.argtypes = [_vp, ctypes.POINTER(Stats)]
    L.octopus_plan_device_bytes.argtypes = [_vp]
    L.octopus_plan_device_bytes.restype = ctypes.c_size_t
    L.octopus_plan_upload.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
    L.octopus_plan_export_mask.argtypes = [_vp, ctypes.c_int32, ctypes.c_int32, _vp]
    L.octopus_plan_export_tiles.argtypes = [_vp, _vp, _vp, _vp, _vp]
    L.octopus_plan_destroy.argtypes = [_vp]
    L.octopus_plan_destroy.restype = None
    L.octopus_fwd_workspace_bytes.argtypes = [_vp, ctypes.c_int, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32]
    L.octopus_fwd_workspace_bytes.restype = ctypes.c_size_t
    L.octopus_bwd_workspace_bytes.argtypes = L.octopus_fwd_workspace_bytes.argtypes
    L.octopus_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.octopus_dag_attn_fwd.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_float, _vp, _vp, _vp, _vp, _vp,
                                       _vp, ctypes.c_size_t, _vp]
    L.octopus_dag_attn_bwd.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_float, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.octopus_dag_attn_bwd_preprocess.argtypes = [_vp, ctypes.c_int, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_int32, _vp, _vp,
                                                  _vp, _vp, ctypes.c_size_t, _vp]
    L.octopus_dag_attn_bwd_dkdv.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_float, _vp, _vp, _vp, _vp,
                                            _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.octopus_dag_attn_bwd_dq.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_float, _vp, _vp, _vp, _vp,
                                          _vp, _vp, ctypes.c_size_t, _vp]
    L.octopus_decode_segments.argtypes = [_vp, ctypes.c_int32, _vp, ctypes.c_int32, _vp, _vp,
                                          ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int32,
                                          ctypes.c_int32, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                          _i32p, _vp, _vp, _i32p]
    L.octopus_decode_workspace_bytes.argtypes = [ctypes.c_int32] * 4
    L.octopus_decode_workspace_bytes.restype = ctypes.c_size_t
    L.octopus_paged_mount_decode.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_float, _vp, _vp, _vp, ctypes.c_int32,
                                             _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp,
                                             ctypes.c_int32, _vp, _vp, _vp, ctypes.c_size_t,
                                             _vp]
    L.octopus_paged_mount_decode_noalloc.argtypes = L.octopus_paged_mount_decode.argtypes[:-3] + [_vp]
    L.octopus_extend_segments.argtypes = [_vp, ctypes.c_int32, _vp, ctypes.c_int32, _vp, _vp,
                                          ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int32,
                                          _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                          _i32p, _vp]
    L.octopus_paged_mount_extend.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_float, _vp, _vp, _vp, ctypes.c_int32,
                                             _vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _vp, _vp, _vp, _vp]
    L.octopus_dag_positions.argtypes = [_vp, ctypes.c_int32, _vp, ctypes.c_int32,
                                        ctypes.c_int32, _vp]
    L.octopus_rope.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                               ctypes.c_float, ctypes.c_int32, _vp, _vp, _vp, _vp]
    L.octopus_rope_workspace_bytes.argtypes = [_vp, ctypes.c_int, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_int32]
    L.octopus_rope_workspace_bytes.restype = ctypes.c_size_t
    L.octopus_dag_attn_fwd_rope.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                            _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.octopus_dag_attn_bwd_rope.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                            ctypes.c_size_t, _vp]
    L.octopus_gdn_workspace_bytes.argtypes = [_vp, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32]
    L.octopus_gdn_workspace_bytes.restype = ctypes.c_size_t
    L.octopus_gated_delta_scan.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                           ctypes.c_size_t, _vp]
    L.octopus_gdn_bwd_workspace_bytes.argtypes = L.octopus_gdn_workspace_bytes.argtypes
    L.octopus_gdn_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.octopus_gated_delta_scan_bwd.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32] + [_vp] * 11 + [_vp,
                                                                                ctypes.c_size_t, _vp]
    L.octopus_gated_delta_scan_save.argtypes = L.octopus_gated_delta_scan.argtypes
    L.octopus_gated_delta_scan_bwd_saved.argtypes = L.octopus_gated_delta_scan_bwd.argtypes
    L.octopus_last_error.restype = ctypes.c_char_p
    L.octopus_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc):
    if rc != OK:
        raise OctopusError(rc, lib().octopus_last_error().decode())


def _np_ptr(a):
    return a.ctypes.data_as(_vp)


def _tables(branches, mounts):
    br = np.ascontiguousarray(np.asarray(branches, dtype=np.int32).reshape(-1, 4))
    mt = np.ascontiguousarray(np.asarray(mounts, dtype=np.int32).reshape(-1, 5))
    return br, mt


# ----------------------------------------------------------------------------- plan

class Plan:
    """A tile plan of one packed tree (host object; ``upload`` puts a copy on the
    device in a caller-owned buffer)."""

    def __init__(self, branches, mounts, total_tokens, kv_tile=64):
        self._h = None
        br, mt = _tables(branches, mounts)
        h = _vp()
        _check(lib().octopus_dag_plan(_np_ptr(br), br.shape[0], _np_ptr(mt), mt.shape[0],
                                      int(total_tokens), int(kv_tile), ctypes.byref(h)))
        self._h = h
        self.T = int(total_tokens)
        self.dev = None

    def __del__(self):
        if getattr(self, "_h", None) is not None and _lib is not None:
            _lib.octopus_plan_destroy(self._h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def positions(self) -> np.ndarray:
        out = np.empty(self.T, dtype=np.int32)
        _check(lib().octopus_plan_positions(self._h, out.ctypes.data_as(_i32p)))
        return out

    def stats(self) -> dict:
        s = Stats()
        _check(lib().octopus_plan_stats_get(self._h, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in Stats._fields_ if f != "reserved"}

    def device_bytes(self) -> int:
        return int(lib().octopus_plan_device_bytes(self._h))

    def export_mask(self, row_lo, row_hi) -> np.ndarray:
        out = np.zeros((row_hi - row_lo, (self.T + 7) // 8), dtype=np.uint8)
        _check(lib().octopus_plan_export_mask(self._h, int(row_lo), int(row_hi), _np_ptr(out)))
        return out

    def tiles(self):
        """``(qt_ptr, kv_tile, mask, rows)``: the forward tile lists and PARTIAL masks."""
        st = self.stats()
        qt_ptr = np.zeros(st["n_q_tiles"] + 1, dtype=np.int32)
        kv = np.zeros(max(st["n_pairs"], 1), dtype=np.int32)
        mk = np.zeros(max(st["n_pairs"], 1), dtype=np.int32)
        rows = np.zeros((max(st["n_partial"], 1), 128), dtype=np.uint64)
        _check(lib().octopus_plan_export_tiles(self._h, _np_ptr(qt_ptr), _np_ptr(kv),
                                               _np_ptr(mk), _np_ptr(rows)))
        n = st["n_pairs"]
        return qt_ptr, kv[:n], mk[:n], rows[:st["n_partial"]]

    def upload(self, device="cuda", buffer=None, sync=True, stream=None):
        """Copy the plan into ``buffer`` (a uint8 CUDA tensor, allocated here if
        ``None``) on ``stream`` (default: the current stream).  With ``sync`` the call
        waits for the copy; otherwise keep this object alive until the stream has
        finished with it."""
        import torch
        n = self.device_bytes()
        mine = buffer is None
        if buffer is None:
            buffer = torch.empty(n, dtype=torch.uint8, device=device)
        if buffer.dtype != torch.uint8 or not buffer.is_cuda or not buffer.is_contiguous():
            raise OctopusError(EINVAL, "plan buffer must be a contiguous uint8 device tensor")
        stream = _stream(stream, buffer.device)
        if mine:
            _owned(stream, buffer)
        _check(lib().octopus_plan_upload(self._h, _vp(buffer.data_ptr()), buffer.numel(),
                                         _vp(stream.cuda_stream)))
        if sync:
            stream.synchronize()
        self.dev = buffer
        return self


# ----------------------------------------------------------------------------- attention

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise OctopusError(EUNSUPPORTED, f"dtype {t.dtype} not supported")


def _stream(stream, device):
    """The stream to enqueue on (the current one if ``stream`` is None)."""
    import torch
    return stream or torch.cuda.current_stream(device)


def _owned(s, *tensors):
    """Tensors this module allocated for work enqueued on ``s``: when ``s`` is not the
    current stream, tell the caching allocator they are in use there, so their memory
    is not handed to other work before ``s`` has finished with it."""
    import torch
    for t in tensors:
        if t is not None and s != torch.cuda.current_stream(t.device):
            t.record_stream(s)


def _need(t, shape, dtype, name):
    if tuple(t.shape) != tuple(shape):
        raise OctopusError(EINVAL, f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise OctopusError(EINVAL, f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_contiguous():
        raise OctopusError(EINVAL, f"{name} must be contiguous")
    if not t.is_cuda:
        raise OctopusError(EINVAL, f"{name} must be a device tensor")


def fwd_workspace_bytes(plan: Plan, dtype_code, Hq, Hkv, D) -> int:
    return int(lib().octopus_fwd_workspace_bytes(plan.handle, dtype_code, Hq, Hkv, D))


def attn_fwd(plan: Plan, q, k, v, scale=None, o=None, lse=None, ws=None, stream=None):
    """Packed-DAG attention forward: returns ``(o [T,Hq,D], lse float32 [Hq,T])``.
    ``ws`` (uint8 device tensor of fwd_workspace_bytes) is allocated when not given."""
    import torch
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    _need(q, (plan.T, Hq, D), q.dtype, "q")
    _need(k, (plan.T, Hkv, D), q.dtype, "k")
    _need(v, (plan.T, Hkv, D), q.dtype, "v")
    s = _stream(stream, q.device)
    mine = []
    if o is None:
        o = torch.empty_like(q)
        mine.append(o)
    if lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
        mine.append(lse)
    _need(o, q.shape, q.dtype, "o")
    _need(lse, (Hq, T), torch.float32, "lse")
    code = _dtype_code(q)
    if ws is None:
        need = fwd_workspace_bytes(plan, code, Hq, Hkv, D)
        ws = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
        mine.append(ws)
    _owned(s, *mine)
    _check(lib().octopus_dag_attn_fwd(plan.handle, code, Hq, Hkv, D, float(scale or 0.0),
                                      q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), None if ws is None else ws.data_ptr(),
                                      0 if ws is None else ws.numel(), _vp(s.cuda_stream)))
    return o, lse


def bwd_workspace_bytes(plan: Plan, dtype_code, Hq, Hkv, D) -> int:
    return int(lib().octopus_bwd_workspace_bytes(plan.handle, dtype_code, Hq, Hkv, D))


def attn_bwd(plan: Plan, q, k, v, o, lse, dout, scale=None, dq=None, dk=None, dv=None,
             ws=None, stream=None):
    """Packed-DAG attention backward: returns ``(dq, dk, dv)``."""
    import torch
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    for t, shp, nm in ((q, (plan.T, Hq, D), "q"), (k, (plan.T, Hkv, D), "k"),
                       (v, (plan.T, Hkv, D), "v"), (o, (plan.T, Hq, D), "o"),
                       (dout, (plan.T, Hq, D), "dout")):
        _need(t, shp, q.dtype, nm)
    _need(lse, (Hq, T), torch.float32, "lse")
    s = _stream(stream, q.device)
    mine = []
    if dq is None:
        dq = torch.empty_like(q)
        mine.append(dq)
    if dk is None:
        dk = torch.empty_like(k)
        mine.append(dk)
    if dv is None:
        dv = torch.empty_like(v)
        mine.append(dv)
    code = _dtype_code(q)
    need = bwd_workspace_bytes(plan, code, Hq, Hkv, D)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        mine.append(ws)
    _owned(s, *mine)
    _check(lib().octopus_dag_attn_bwd(plan.handle, code, Hq, Hkv, D, float(scale or 0.0),
                                      q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                      dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
                                      _vp(s.cuda_stream)))
    return dq, dk, dv


def attn_bwd_phase(phase, plan: Plan, q, k, v, o, lse, dout, ws, dq=None, dk=None, dv=None,
                   scale=None, stream=None):
    """One backward phase: ``"preprocess"`` (Delta into ``ws``), ``"dkdv"`` or
    ``"dq"``; the output tensors must be given."""
    import torch
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    code = _dtype_code(q)
    s = _vp((stream or torch.cuda.current_stream(q.device)).cuda_stream)
    L = lib()
    sc = float(scale or 0.0)
    if phase == "preprocess":
        rc = L.octopus_dag_attn_bwd_preprocess(plan.handle, code, Hq, Hkv, D, o.data_ptr(),
                                               lse.data_ptr(), dout.data_ptr(), ws.data_ptr(),
                                               ws.numel(), s)
    elif phase == "dkdv":
        rc = L.octopus_dag_attn_bwd_dkdv(plan.handle, code, Hq, Hkv, D, sc, q.data_ptr(),
                                         k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                         dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                                         ws.numel(), s)
    elif phase == "dq":
        rc = L.octopus_dag_attn_bwd_dq(plan.handle, code, Hq, Hkv, D, sc, q.data_ptr(),
                                       k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                       dq.data_ptr(), ws.data_ptr(), ws.numel(), s)
    else:
        raise ValueError(phase)
    _check(rc)


# ----------------------------------------------------------------------------- rope

def dag_positions(branches, mounts, total_tokens) -> np.ndarray:
    """Positions of the packed tokens (host int32), no tile plan built."""
    br, mt = _tables(branches, mounts)
    out = np.zeros(max(int(total_tokens), 1), dtype=np.int32)
    _check(lib().octopus_dag_positions(_np_ptr(br), br.shape[0], _np_ptr(mt), mt.shape[0],
                                       int(total_tokens), _np_ptr(out)))
    return out[:int(total_tokens)]


def rope(x, pos, base=10000.0, inverse=False, out=None, stream=None):
    """Rotate-half RoPE of ``x [rows, H, D]`` (device) at ``pos`` (device int32
    ``[rows]``); ``out`` may be ``x``."""
    import torch
    rows, H, D = x.shape
    if not (x.is_cuda and x.is_contiguous()):
        raise OctopusError(EINVAL, "x must be a contiguous device tensor")
    if pos.dtype != torch.int32 or not pos.is_cuda or pos.numel() != rows:
        raise OctopusError(EINVAL, "pos must be a device int32 tensor with one entry per row")
    s = _stream(stream, x.device)
    if out is None:
        out = torch.empty_like(x)
        _owned(s, out)
    _need(out, x.shape, x.dtype, "out")
    _check(lib().octopus_rope(_dtype_code(x), rows, H, D, float(base), 1 if inverse else 0,
                              pos.data_ptr(), x.data_ptr(), out.data_ptr(), _vp(s.cuda_stream)))
    return out


def rope_workspace_bytes(plan: Plan, dtype_code, Hq, Hkv, D) -> int:
    return int(lib().octopus_rope_workspace_bytes(plan.handle, dtype_code, Hq, Hkv, D))


def attn_fwd_rope(plan: Plan, q, k, v, base=10000.0, scale=None, o=None, lse=None, ws=None,
                  stream=None):
    """Forward with unrotated Q and K, turned at the plan's positions first."""
    import torch
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    _need(q, (plan.T, Hq, D), q.dtype, "q")
    _need(k, (plan.T, Hkv, D), q.dtype, "k")
    _need(v, (plan.T, Hkv, D), q.dtype, "v")
    s = _stream(stream, q.device)
    mine = []
    if o is None:
        o = torch.empty_like(q)
        mine.append(o)
    if lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
        mine.append(lse)
    code = _dtype_code(q)
    if ws is None:
        need = rope_workspace_bytes(plan, code, Hq, Hkv, D) + fwd_workspace_bytes(plan, code,
                                                                                Hq, Hkv, D)
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        mine.append(ws)
    _owned(s, *mine)
    _check(lib().octopus_dag_attn_fwd_rope(plan.handle, code, Hq, Hkv, D, float(scale or 0.0),
                                           float(base), q.data_ptr(), k.data_ptr(),
                                           v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                           ws.data_ptr(), ws.numel(), _vp(s.cuda_stream)))
    return o, lse


def attn_bwd_rope(plan: Plan, q, k, v, o, lse, dout, base=10000.0, scale=None, dq=None,
                  dk=None, dv=None, ws=None, stream=None):
    """Backward with unrotated Q and K: returns gradients with respect to them."""
    import torch
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    for t, shp, nm in ((q, (plan.T, Hq, D), "q"), (k, (plan.T, Hkv, D), "k"),
                       (v, (plan.T, Hkv, D), "v"), (o, (plan.T, Hq, D), "o"),
                       (dout, (plan.T, Hq, D), "dout")):
        _need(t, shp, q.dtype, nm)
    s = _stream(stream, q.device)
    mine = []
    if dq is None:
        dq = torch.empty_like(q)
        mine.append(dq)
    if dk is None:
        dk = torch.empty_like(k)
        mine.append(dk)
    if dv is None:
        dv = torch.empty_like(v)
        mine.append(dv)
    code = _dtype_code(q)
    if ws is None:
        need = rope_workspace_bytes(plan, code, Hq, Hkv, D) + bwd_workspace_bytes(plan, code,
                                                                                Hq, Hkv, D)
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        mine.append(ws)
    _owned(s, *mine)
    _check(lib().octopus_dag_attn_bwd_rope(plan.handle, code, Hq, Hkv, D, float(scale or 0.0),
                                           float(base), q.data_ptr(), k.data_ptr(),
                                           v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                           dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                           dv.data_ptr(), ws.data_ptr(), ws.numel(),
                                           _vp(s.cuda_stream)))
    return dq, dk, dv


# ----------------------------------------------------------------------------- scan

def gdn_workspace_bytes(plan: Plan, H, Dk=128, Dv=128) -> int:
    return int(lib().octopus_gdn_workspace_bytes(plan.handle, H, Dk, Dv))


def gated_delta_scan(plan: Plan, q, k, v, alpha, beta, o=None, ws=None, stream=None):
    """Branch-aware gated delta-rule scan: ``q, k [T,H,Dk]``, ``v [T,H,Dv]`` bf16,
    ``alpha, beta`` float32 ``[T,H]``; returns ``o [T,H,Dv]``."""
    import torch
    T, H, Dk = q.shape
    Dv = v.shape[2]
    _need(q, (plan.T, H, Dk), q.dtype, "q")
    _need(k, (plan.T, H, Dk), q.dtype, "k")
    _need(v, (plan.T, H, Dv), q.dtype, "v")
    _need(alpha, (plan.T, H), torch.float32, "alpha")
    _need(beta, (plan.T, H), torch.float32, "beta")
    s = _stream(stream, q.device)
    mine = []
    if o is None:
        o = torch.empty_like(v)
        mine.append(o)
    if ws is None:
        ws = torch.empty(max(gdn_workspace_bytes(plan, H, Dk, Dv), 16), dtype=torch.uint8,
                         device=q.device)
        mine.append(ws)
    _owned(s, *mine)
    _check(lib().octopus_gated_delta_scan(plan.handle, _dtype_code(q), H, Dk, Dv, q.data_ptr(),
                                          k.data_ptr(), v.data_ptr(), alpha.data_ptr(),
                                          beta.data_ptr(), o.data_ptr(), ws.data_ptr(),
                                          ws.numel(), _vp(s.cuda_stream)))
    return o


def gdn_bwd_workspace_bytes(plan: Plan, H, Dk=128, Dv=128) -> int:
    return int(lib().octopus_gdn_bwd_workspace_bytes(plan.handle, H, Dk, Dv))


def gated_delta_scan_bwd(plan: Plan, q, k, v, alpha, beta, dout, dq=None, dk=None, dv=None,
                         dalpha=None, dbeta=None, ws=None, stream=None):
    """Backward of ``gated_delta_scan``: returns ``(dq, dk, dv, dalpha, dbeta)``."""
    import torch
    T, H, Dk = q.shape
    Dv = v.shape[2]
    _need(q, (plan.T, H, Dk), q.dtype, "q")
    _need(k, (plan.T, H, Dk), q.dtype, "k")
    _need(v, (plan.T, H, Dv), q.dtype, "v")
    _need(dout, (plan.T, H, Dv), q.dtype, "dout")
    _need(alpha, (plan.T, H), torch.float32, "alpha")
    _need(beta, (plan.T, H), torch.float32, "beta")
    s = _stream(stream, q.device)
    mine = []
    if dq is None:
        dq = torch.empty_like(q)
        mine.append(dq)
    if dk is None:
        dk = torch.empty_like(k)
        mine.append(dk)
    if dv is None:
        dv = torch.empty_like(v)
        mine.append(dv)
    if dalpha is None:
        dalpha = torch.empty_like(alpha)
        mine.append(dalpha)
    if dbeta is None:
        dbeta = torch.empty_like(beta)
        mine.append(dbeta)
    if ws is None:
        ws = torch.empty(max(gdn_bwd_workspace_bytes(plan, H, Dk, Dv), 16), dtype=torch.uint8,
                         device=q.device)
        mine.append(ws)
    _owned(s, *mine)
    _check(lib().octopus_gated_delta_scan_bwd(
        plan.handle, _dtype_code(q), H, Dk, Dv, q.data_ptr(), k.data_ptr(), v.data_ptr(),
        alpha.data_ptr(), beta.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
        dv.data_ptr(), dalpha.data_ptr(), dbeta.data_ptr(), ws.data_ptr(), ws.numel(),
        _vp(s.cuda_stream)))
    return dq, dk, dv, dalpha, dbeta


def gated_delta_scan_save(plan: Plan, q, k, v, alpha, beta, o=None, ws=None, stream=None):
    """``gated_delta_scan`` that also keeps, in ``ws`` (``gdn_bwd_workspace_bytes``), what
    ``gated_delta_scan_bwd_saved`` reads: returns ``(o, ws)``.  Keep ``ws`` and the inputs
    unchanged until the backward has run."""
    import torch
    T, H, Dk = q.shape
    Dv = v.shape[2]
    _need(q, (plan.T, H, Dk), q.dtype, "q")
    _need(k, (plan.T, H, Dk), q.dtype, "k")
    _need(v, (plan.T, H, Dv), q.dtype, "v")
    _need(alpha, (plan.T, H), torch.float32, "alpha")
    _need(beta, (plan.T, H), torch.float32, "beta")
    s = _stream(stream, q.device)
    mine = []
    if o is None:
        o = torch.empty_like(v)
        mine.append(o)
    if ws is None:
        ws = torch.empty(max(gdn_bwd_workspace_bytes(plan, H, Dk, Dv), 16), dtype=torch.uint8,
                         device=q.device)
        mine.append(ws)
    _owned(s, *mine)
    _check(lib().octopus_gated_delta_scan_save(plan.handle, _dtype_code(q), H, Dk, Dv,
                                               q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                               alpha.data_ptr(), beta.data_ptr(), o.data_ptr(),
                                               ws.data_ptr(), ws.numel(), _vp(s.cuda_stream)))
    return o, ws


def gated_delta_scan_bwd_saved(plan: Plan, q, k, v, alpha, beta, dout, ws, dq=None, dk=None,
                               dv=None, dalpha=None, dbeta=None, stream=None):
    """Backward of ``gated_delta_scan_save`` from the workspace it filled: returns
    ``(dq, dk, dv, dalpha, dbeta)``."""
    import torch
    T, H, Dk = q.shape
    Dv = v.shape[2]
    _need(q, (plan.T, H, Dk), q.dtype, "q")
    _need(k, (plan.T, H, Dk), q.dtype, "k")
    _need(v, (plan.T, H, Dv), q.dtype, "v")
    _need(dout, (plan.T, H, Dv), q.dtype, "dout")
    _need(alpha, (plan.T, H), torch.float32, "alpha")
    _need(beta, (plan.T, H), torch.float32, "beta")
    s = _stream(stream, q.device)
    outs = []
    for t, like in ((dq, q), (dk, k), (dv, v), (dalpha, alpha), (dbeta, beta)):
        outs.append(torch.empty_like(like) if t is None else t)
    _owned(s, *[o for o, t in zip(outs, (dq, dk, dv, dalpha, dbeta)) if t is None])
    dq, dk, dv, dalpha, dbeta = outs
    _check(lib().octopus_gated_delta_scan_bwd_saved(
        plan.handle, _dtype_code(q), H, Dk, Dv, q.data_ptr(), k.data_ptr(), v.data_ptr(),
        alpha.data_ptr(), beta.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
        dv.data_ptr(), dalpha.data_ptr(), dbeta.data_ptr(), ws.data_ptr(), ws.numel(),
        _vp(s.cuda_stream)))
    return dq, dk, dv, dalpha, dbeta


# ----------------------------------------------------------------------------- decode

def decode_segments(branches, mounts, page_ptr, pages, page_size, n_pages, cursors,
                    share=False):
    """Host segment builder.  Returns int32 arrays ``(seg_ptr, seg_page, seg_lo,
    seg_hi)`` with one list per cursor (its whole context); with ``share``, also
    ``(grp_ptr, grp_cur)``: each cursor's list then holds only what it does not inherit,
    followed by one list per group of cursors forked from the same (parent, fork) with
    the context they all inherit (``seg_ptr`` has ``B + n_groups + 1`` entries)."""
    br, mt = _tables(branches, mounts)
    pp = np.ascontiguousarray(page_ptr, dtype=np.int32)
    pg = np.ascontiguousarray(pages, dtype=np.int32)
    cur = np.ascontiguousarray(cursors, dtype=np.int32)
    B = cur.shape[0]
    n = ctypes.c_int32(0)
    ng = ctypes.c_int32(0)
    L = lib()
    args = [_np_ptr(br), br.shape[0], _np_ptr(mt), mt.shape[0], _np_ptr(pp), _np_ptr(pg),
            int(page_size), int(n_pages), _np_ptr(cur), B, 1 if share else 0]
    rc = L.octopus_decode_segments(*args, None, None, None, None, 0, ctypes.byref(n), None,
                                   None, ctypes.byref(ng))
    if rc not in (OK, EWORKSPACE):
        _check(rc)
    cap = n.value
    sp = np.zeros(2 * B + 1, dtype=np.int32)
    gp = np.zeros(B + 1, dtype=np.int32)
    gc = np.zeros(max(B, 1), dtype=np.int32)
    out = [np.zeros(max(cap, 1), dtype=np.int32) for _ in range(3)]
    _check(L.octopus_decode_segments(*args, _np_ptr(sp), _np_ptr(out[0]), _np_ptr(out[1]),
                                     _np_ptr(out[2]), cap, ctypes.byref(n), _np_ptr(gp),
                                     _np_ptr(gc), ctypes.byref(ng)))
    segs = (out[0][:cap], out[1][:cap], out[2][:cap])
    if not share:
        return (sp[:B + 1],) + segs
    return (sp[:B + ng.value + 1],) + segs + (gp[:ng.value + 1], gc[:B])


def decode_workspace_bytes(B, Hq, D, n_split) -> int:
    return int(lib().octopus_decode_workspace_bytes(B, Hq, D, n_split))


def paged_mount_decode(q, k_pool, v_pool, seg_ptr, seg_page, seg_lo, seg_hi, grp_ptr=None,
                       grp_cur=None, n_split=16, scale=None, o=None, lse=None, ws=None,
                       stream=None):
    """One-token attention of every cursor over its segments (device int32 tensors, as
    ``decode_segments`` returns them; ``grp_ptr``/``grp_cur`` with ``share``).
    Returns ``(o [B,Hq,D], lse float32 [B,Hq])``."""
    import torch
    B, Hq, D = q.shape
    n_pages, Hkv, page_size, _ = k_pool.shape
    _need(q, (B, Hq, D), q.dtype, "q")
    _need(k_pool, (n_pages, Hkv, page_size, D), q.dtype, "k_pool")
    _need(v_pool, (n_pages, Hkv, page_size, D), q.dtype, "v_pool")
    arrays = [(seg_ptr, "seg_ptr"), (seg_page, "seg_page"), (seg_lo, "seg_lo"),
              (seg_hi, "seg_hi")]
    if (grp_ptr is None) != (grp_cur is None):
        raise OctopusError(EINVAL, "grp_ptr and grp_cur go together")
    n_groups = 0
    if grp_ptr is not None:
        arrays += [(grp_ptr, "grp_ptr"), (grp_cur, "grp_cur")]
        n_groups = grp_ptr.numel() - 1
        if grp_cur.numel() != B:
            raise OctopusError(EINVAL, "grp_cur must have B entries")
    for t, nm in arrays:
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise OctopusError(EINVAL, f"{nm} must be a contiguous int32 device tensor")
    if seg_ptr.numel() != B + n_groups + 1:
        raise OctopusError(EINVAL, "seg_ptr must have B + n_groups + 1 entries")
    s = _stream(stream, q.device)
    mine = []
    if o is None:
        o = torch.empty_like(q)
        mine.append(o)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        mine.append(lse)
    need = decode_workspace_bytes(B, Hq, D, n_split)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        mine.append(ws)
    _owned(s, *mine)
    gp = grp_ptr.data_ptr() if grp_ptr is not None else None
    gc = grp_cur.data_ptr() if grp_cur is not None else None
    _check(lib().octopus_paged_mount_decode(
        _dtype_code(q), B, Hq, Hkv, D, page_size, float(scale or 0.0), q.data_ptr(),
        k_pool.data_ptr(), v_pool.data_ptr(), n_pages, seg_ptr.data_ptr(), seg_page.data_ptr(),
        seg_lo.data_ptr(), seg_hi.data_ptr(), n_groups, gp, gc, int(n_split), o.data_ptr(),
        lse.data_ptr(), ws.data_ptr(), ws.numel(), _vp(s.cuda_stream)))
    return o, lse


def paged_mount_decode_noalloc(q, k_pool, v_pool, seg_ptr, seg_page, seg_lo, seg_hi,
                               grp_ptr=None, grp_cur=None, n_split=16, scale=None, o=None,
                               lse=None, stream=None):
    """``paged_mount_decode`` through the entry point that allocates no device memory:
    the partial states live in the library's per-GPU scratch array (at most
    ``DECODE_SCRATCH_BYTES``; calls that overlap on one GPU race).  Pass ``o`` and
    ``lse`` to allocate nothing here either."""
    import torch
    B, Hq, D = q.shape
    n_pages, Hkv, page_size, _ = k_pool.shape
    _need(q, (B, Hq, D), q.dtype, "q")
    _need(k_pool, (n_pages, Hkv, page_size, D), q.dtype, "k_pool")
    _need(v_pool, (n_pages, Hkv, page_size, D), q.dtype, "v_pool")
    arrays = [(seg_ptr, "seg_ptr"), (seg_page, "seg_page"), (seg_lo, "seg_lo"),
              (seg_hi, "seg_hi")]
    if (grp_ptr is None) != (grp_cur is None):
        raise OctopusError(EINVAL, "grp_ptr and grp_cur go together")
    n_groups = 0
    if grp_ptr is not None:
        arrays += [(grp_ptr, "grp_ptr"), (grp_cur, "grp_cur")]
        n_groups = grp_ptr.numel() - 1
        if grp_cur.numel() != B:
            raise OctopusError(EINVAL, "grp_cur must have B entries")
    for t, nm in arrays:
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise OctopusError(EINVAL, f"{nm} must be a contiguous int32 device tensor")
    if seg_ptr.numel() != B + n_groups + 1:
        raise OctopusError(EINVAL, "seg_ptr must have B + n_groups + 1 entries")
    s = _stream(stream, q.device)
    mine = []
    if o is None:
        o = torch.empty_like(q)
        mine.append(o)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        mine.append(lse)
    _need(o, q.shape, q.dtype, "o")
    _need(lse, (B, Hq), torch.float32, "lse")
    _owned(s, *mine)
    gp = grp_ptr.data_ptr() if grp_ptr is not None else None
    gc = grp_cur.data_ptr() if grp_cur is not None else None
    _check(lib().octopus_paged_mount_decode_noalloc(
        _dtype_code(q), B, Hq, Hkv, D, page_size, float(scale or 0.0), q.data_ptr(),
        k_pool.data_ptr(), v_pool.data_ptr(), n_pages, seg_ptr.data_ptr(), seg_page.data_ptr(),
        seg_lo.data_ptr(), seg_hi.data_ptr(), n_groups, gp, gc, int(n_split), o.data_ptr(),
        lse.data_ptr(), _vp(s.cuda_stream)))
    return o, lse


# ----------------------------------------------------------------------------- extend

def extend_segments(branches, mounts, page_ptr, pages, page_size, n_pages, cursors, n_new):
    """Host segment builder for extend: returns int32 arrays ``(seg_ptr, seg_page, seg_lo,
    seg_hi, seg_thr, seg_causal, first_off)``."""
    br, mt = _tables(branches, mounts)
    pp = np.ascontiguousarray(page_ptr, dtype=np.int32)
    pg = np.ascontiguousarray(pages, dtype=np.int32)
    cur = np.ascontiguousarray(cursors, dtype=np.int32)
    nn = np.ascontiguousarray(n_new, dtype=np.int32)
    B = cur.shape[0]
    if nn.shape != (B,):
        raise OctopusError(EINVAL, "n_new must have one entry per cursor")
    n = ctypes.c_int32(0)
    L = lib()
    args = [_np_ptr(br), br.shape[0], _np_ptr(mt), mt.shape[0], _np_ptr(pp), _np_ptr(pg),
            int(page_size), int(n_pages), _np_ptr(cur), B, _np_ptr(nn)]
    rc = L.octopus_extend_segments(*args, None, None, None, None, None, None, 0,
                                   ctypes.byref(n), None)
    if rc not in (OK, EWORKSPACE):
        _check(rc)
    cap = n.value
    sp = np.zeros(B + 1, dtype=np.int32)
    fo = np.zeros(max(B, 1), dtype=np.int32)
    out = [np.zeros(max(cap, 1), dtype=np.int32) for _ in range(5)]
    _check(L.octopus_extend_segments(*args, _np_ptr(sp), *[_np_ptr(a) for a in out], cap,
                                     ctypes.byref(n), _np_ptr(fo)))
    return (sp,) + tuple(a[:cap] for a in out) + (fo[:B],)


def paged_mount_extend(q, k_pool, v_pool, q_ptr, max_new, first_off, seg_ptr, seg_page,
                       seg_lo, seg_hi, seg_thr, seg_causal, scale=None, o=None, lse=None,
                       stream=None):
    """Attention of every cursor's new tokens (rows ``q_ptr[c] .. q_ptr[c+1]-1`` of
    ``q [n_rows, Hq, D]``, at most ``max_new`` per cursor) over their paged context;
    index arrays are contiguous int32 device tensors as ``extend_segments`` returns
    them.  Returns ``(o [n_rows, Hq, D], lse float32 [n_rows, Hq])``."""
    import torch
    n_rows, Hq, D = q.shape
    n_pages, Hkv, page_size, _ = k_pool.shape
    _need(q, (n_rows, Hq, D), q.dtype, "q")
    _need(k_pool, (n_pages, Hkv, page_size, D), q.dtype, "k_pool")
    _need(v_pool, (n_pages, Hkv, page_size, D), q.dtype, "v_pool")
    for t, nm in ((q_ptr, "q_ptr"), (first_off, "first_off"), (seg_ptr, "seg_ptr"),
                  (seg_page, "seg_page"), (seg_lo, "seg_lo"), (seg_hi, "seg_hi"),
                  (seg_thr, "seg_thr"), (seg_causal, "seg_causal")):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise OctopusError(EINVAL, f"{nm} must be a contiguous int32 device tensor")
    B = q_ptr.numel() - 1
    if first_off.numel() != B or seg_ptr.numel() != B + 1:
        raise OctopusError(EINVAL, "first_off and seg_ptr must match q_ptr's cursor count")
    s = _stream(stream, q.device)
    mine = []
    if o is None:
        o = torch.empty_like(q)
        mine.append(o)
    if lse is None:
        lse = torch.empty((n_rows, Hq), dtype=torch.float32, device=q.device)
        mine.append(lse)
    _owned(s, *mine)
    _check(lib().octopus_paged_mount_extend(
        _dtype_code(q), B, Hq, Hkv, D, page_size, float(scale or 0.0), q.data_ptr(),
        k_pool.data_ptr(), v_pool.data_ptr(), n_pages, q_ptr.data_ptr(), int(max_new),
        first_off.data_ptr(), seg_ptr.data_ptr(), seg_page.data_ptr(), seg_lo.data_ptr(),
        seg_hi.data_ptr(), seg_thr.data_ptr(), seg_causal.data_ptr(), o.data_ptr(),
        lse.data_ptr(), _vp(s.cuda_stream)))
    return o, lse


def default_scale(D) -> float:
    return 1.0 / math.sqrt(D)
