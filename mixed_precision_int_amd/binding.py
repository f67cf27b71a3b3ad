"""Thin Python binding of libaq.so (include/aq.h).

Argument marshalling only: every step of the linear layer runs in the HIP
kernels of libaq.so.  PyTorch provides device memory and the current stream.
The functions keep the C names; they take torch tensors and raise AqError on
a non-zero status.  There is no fallback: without the built library every
call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libaq.so")

AQ_PHASE_DECODE = 0
AQ_PHASE_PREFILL = 1
AQ_PHASE_PREFILL_GROUPED = 2
AQ_PHASE_DECODE_TRANSFORMED = 3
AQ_PHASE_DECODE_FP32 = 4

STATUS = {0: "AQ_OK", -1: "AQ_ERR_NULL", -2: "AQ_ERR_SHAPE", -3: "AQ_ERR_TILE", -4: "AQ_ERR_MAP",
          -5: "AQ_ERR_ALIGN", -6: "AQ_ERR_WORKSPACE", -7: "AQ_ERR_HIP", -8: "AQ_ERR_ARG"}

# Every symbol include/aq.h declares.
EXPORTS = ["aq_abi_version", "aq_status_string", "aq_labels_from_map", "aq_plan_pack",
           "aq_pack_weights", "aq_quant_act", "aq_workspace_bytes", "aq_decode_split",
           "aq_linear_decode", "aq_linear_prefill", "aq_linear_tile_partials",
           "aq_quant_act_grouped", "aq_linear_decode_grouped", "aq_linear_prefill_grouped",
           "aq_linear_tile_partials_grouped", "aq_pack_weights_mse",
           "aq_transform_rows", "aq_transform_out", "aq_transform_weights", "aq_quant_act_transformed",
           "aq_prefill_prepare", "aq_linear_prefill_prepared", "aq_linear_prefill_transformed",
           "aq_act_group_shape", "aq_linear_decode_noalloc", "aq_linear_decode_transformed",
           "aq_linear_decode_fp32"]


class AqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_status_text(status)})")


class AqPlan(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("K", ctypes.c_int32), ("bN", ctypes.c_int32),
                ("bK", ctypes.c_int32), ("R", ctypes.c_int32), ("C", ctypes.c_int32),
                ("T4", ctypes.c_int32), ("T8", ctypes.c_int32),
                ("labels_bytes", ctypes.c_size_t), ("labels_alloc", ctypes.c_size_t),
                ("offs_bytes", ctypes.c_size_t),
                ("w4_bytes", ctypes.c_size_t), ("w8_bytes", ctypes.c_size_t),
                ("s4_bytes", ctypes.c_size_t), ("s8_bytes", ctypes.c_size_t),
                ("meta_bytes", ctypes.c_size_t)]


class AqPacked(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("K", ctypes.c_int32), ("bN", ctypes.c_int32),
                ("bK", ctypes.c_int32), ("T4", ctypes.c_int32), ("T8", ctypes.c_int32),
                ("labels", ctypes.c_void_p), ("row_off4", ctypes.c_void_p),
                ("row_off8", ctypes.c_void_p), ("w4", ctypes.c_void_p), ("w8", ctypes.c_void_p),
                ("s4", ctypes.c_void_p), ("s8", ctypes.c_void_p), ("meta_host", ctypes.c_void_p)]


class AqTransformTables(ctypes.Structure):
    _fields_ = [("perm", (ctypes.c_uint8 * 64) * 6), ("dl", (ctypes.c_int8 * 64) * 6),
                ("dr", (ctypes.c_int8 * 64) * 6)]


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libaq.so; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mixed_precision_int_amd.build` (no fallback exists)")
    # PyTorch ships its own HIP runtime under the same soname; it must be the
    # one in the process before libaq.so resolves its dependency, so that
    # torch streams and allocations are valid inside the library.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "aq_abi_version": (i32, []),
        "aq_status_string": (ctypes.c_char_p, [i32]),
        "aq_labels_from_map": (i32, [vp, i32, i32, vp]),
        "aq_plan_pack": (i32, [i32, i32, i32, i32, vp, ctypes.POINTER(AqPlan)]),
        "aq_pack_weights": (i32, [vp, vp, ctypes.POINTER(AqPacked), vp]),
        "aq_quant_act": (i32, [vp, i32, i32, vp, vp, vp]),
        "aq_workspace_bytes": (sz, [ctypes.POINTER(AqPacked), i32, i32, i32]),
        "aq_decode_split": (i32, [ctypes.POINTER(AqPacked), i32]),
        "aq_linear_decode": (i32, [ctypes.POINTER(AqPacked), vp, vp, i32, vp, vp, i32, vp, sz, vp]),
        "aq_linear_prefill": (i32, [ctypes.POINTER(AqPacked), vp, vp, i32, vp, vp, vp, sz, vp]),
        "aq_linear_decode_noalloc": (i32, [ctypes.POINTER(AqPacked), vp, vp, i32, vp, vp, i32, vp]),
        "aq_linear_decode_fp32": (i32, [ctypes.POINTER(AqPacked), vp, i32, vp, vp, i32, vp, sz, vp]),
        "aq_linear_tile_partials": (i32, [ctypes.POINTER(AqPacked), vp, i32, i32, vp, vp, sz, vp]),
        "aq_quant_act_grouped": (i32, [vp, i32, i32, vp, vp, vp]),
        "aq_act_group_shape": (i32, [i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                     ctypes.POINTER(i32)]),
        "aq_pack_weights_mse": (i32, [vp, vp, ctypes.POINTER(AqPacked), vp]),
        "aq_linear_decode_grouped": (i32, [ctypes.POINTER(AqPacked), vp, vp, i32, vp, vp, i32, vp, sz, vp]),
        "aq_linear_prefill_grouped": (i32, [ctypes.POINTER(AqPacked), vp, vp, i32, vp, vp, vp, sz, vp]),
        "aq_linear_tile_partials_grouped": (i32, [ctypes.POINTER(AqPacked), vp, i32, vp, vp, sz, vp]),
        "aq_transform_rows": (i32, [vp, i32, i32, vp, ctypes.POINTER(AqTransformTables), vp, vp]),
        "aq_transform_out": (i32, [vp, i32, i32, vp, ctypes.POINTER(AqTransformTables), vp, vp, vp]),
        "aq_prefill_prepare": (i32, [ctypes.POINTER(AqPacked), vp, sz, vp]),
        "aq_linear_prefill_transformed": (i32, [ctypes.POINTER(AqPacked), vp, vp, i32, vp, vp,
                                                ctypes.POINTER(AqTransformTables), vp, vp, sz, vp]),
        "aq_linear_prefill_prepared": (i32, [ctypes.POINTER(AqPacked), vp, vp, i32, vp, vp, vp, sz, vp]),
        "aq_linear_decode_transformed": (i32, [ctypes.POINTER(AqPacked), vp, vp, i32, vp, vp,
                                               ctypes.POINTER(AqTransformTables), vp, i32, vp, sz, vp]),
        "aq_quant_act_transformed": (i32, [vp, i32, i32, vp, ctypes.POINTER(AqTransformTables), vp, vp, vp]),
        "aq_transform_weights": (i32, [vp, i32, i32, vp, vp, ctypes.POINTER(AqTransformTables), vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = L
    return L


def _status_text(status: int) -> str:
    try:
        return lib().aq_status_string(status).decode()
    except Exception:  # pragma: no cover - only when the library is absent
        return "?"


def _check(status: int, where: str) -> None:
    if status != 0:
        raise AqError(status, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------- host calls

def aq_abi_version() -> int:
    return lib().aq_abi_version()


def aq_labels_from_map(zmap: np.ndarray) -> np.ndarray:
    """Labels (1 = INT4, LSB first) of an [R, C] map of 4 / 8."""
    z = np.ascontiguousarray(zmap, dtype=np.uint8)
    R, C = z.shape
    out = np.zeros((R * C + 7) // 8, dtype=np.uint8)
    _check(lib().aq_labels_from_map(z.ctypes.data, R, C, out.ctypes.data), "aq_labels_from_map")
    return out


def aq_plan_pack(N: int, K: int, bN: int, bK: int, labels: np.ndarray) -> AqPlan:
    lab = np.ascontiguousarray(labels, dtype=np.uint8)
    plan = AqPlan()
    _check(lib().aq_plan_pack(N, K, bN, bK, lab.ctypes.data, ctypes.byref(plan)), "aq_plan_pack")
    return plan


# ---------------------------------------------------------------- device calls

@dataclass
class PackedWeights:
    """Device buffers of one packed projection and the C descriptor over them."""
    plan: AqPlan
    labels_host: np.ndarray
    labels: object
    row_off4: object
    row_off8: object
    w4: object
    w8: object
    s4: object
    s8: object
    desc: AqPacked
    meta_host: np.ndarray | None = None  # host metadata image (decode passes it inline)

    @property
    def N(self):
        return self.plan.N

    @property
    def K(self):
        return self.plan.K

    def nbytes(self) -> int:
        p = self.plan
        return int(p.labels_bytes + 2 * p.offs_bytes + p.w4_bytes + p.w8_bytes + p.s4_bytes + p.s8_bytes)


def _dev_bytes(n: int, device):
    import torch
    # at least 16 bytes so that every pointer is valid and aligned
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device=device)


def aq_alloc_packed(plan: AqPlan, labels: np.ndarray, device="cuda") -> PackedWeights:
    t = dict(labels=_dev_bytes(plan.labels_alloc, device), row_off4=_dev_bytes(plan.offs_bytes, device),
             row_off8=_dev_bytes(plan.offs_bytes, device), w4=_dev_bytes(plan.w4_bytes, device),
             w8=_dev_bytes(plan.w8_bytes, device), s4=_dev_bytes(plan.s4_bytes, device),
             s8=_dev_bytes(plan.s8_bytes, device))
    meta = np.zeros(max(int(plan.meta_bytes) // 4, 1), dtype=np.uint32)  # [R][6] when C <= 128
    d = AqPacked(plan.N, plan.K, plan.bN, plan.bK, plan.T4, plan.T8,
                 *(t[k].data_ptr() for k in ("labels", "row_off4", "row_off8", "w4", "w8", "s4", "s8")),
                 meta.ctypes.data)
    return PackedWeights(plan=plan, labels_host=np.ascontiguousarray(labels, dtype=np.uint8), desc=d,
                         meta_host=meta, **t)


def aq_pack_weights(W, labels: np.ndarray, bN: int = 64, bK: int = 128, stream=None,
                    mse: bool = False) -> PackedWeights:
    """Quantize and pack W (device FP32 [N, K]) under the given labels; with
    mse=True the weight scales are eq. 7's fitted scales (aq_pack_weights_mse)."""
    N, K = W.shape
    lab = np.ascontiguousarray(labels, dtype=np.uint8)
    plan = aq_plan_pack(N, K, bN, bK, lab)
    pw = aq_alloc_packed(plan, lab, W.device)
    fn = lib().aq_pack_weights_mse if mse else lib().aq_pack_weights
    _check(fn(ctypes.c_void_p(W.data_ptr()), lab.ctypes.data, ctypes.byref(pw.desc), _stream(stream)),
           "aq_pack_weights_mse" if mse else "aq_pack_weights")
    return pw


def aq_quant_act(X, qx=None, sx=None, stream=None):
    """INT8 codes [M, K] and FP32 scales [M] of device FP32 X [M, K]."""
    import torch
    M, K = X.shape
    if qx is None:
        qx = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if sx is None:
        sx = torch.empty((M,), dtype=torch.float32, device=X.device)
    _check(lib().aq_quant_act(ctypes.c_void_p(X.data_ptr()), M, K, ctypes.c_void_p(qx.data_ptr()),
                              ctypes.c_void_p(sx.data_ptr()), _stream(stream)), "aq_quant_act")
    return qx, sx


def aq_workspace_bytes(pw: PackedWeights, M: int, phase: int, split: int = 0) -> int:
    return int(lib().aq_workspace_bytes(ctypes.byref(pw.desc), M, phase, split))


def aq_decode_split(pw: PackedWeights, M: int) -> int:
    return int(lib().aq_decode_split(ctypes.byref(pw.desc), M))


# Decode workspaces, one per (device, stream), grown on demand.  Allocated
# zeroed; every decode call leaves its arrival counters at zero again, so a
# workspace is reused by the calls of its stream (which never overlap).
_DECODE_WS: dict = {}


def decode_workspace(nbytes: int, device, stream=None):
    """A zero-initialized decode workspace of at least nbytes for the stream."""
    import torch
    st = torch.cuda.current_stream(device) if stream is None else stream
    key = (str(torch.device(device)), st.cuda_stream)
    ws = _DECODE_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            st.synchronize()  # the old buffer may still be in use on its stream
        ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        torch.cuda.current_stream(device).synchronize()
        _DECODE_WS[key] = ws
    return ws


def aq_linear_decode(pw: PackedWeights, qx, sx, bias=None, split: int = 0, out=None, ws=None,
                     stream=None):
    """Decode-phase linear: FP32 Y [M, N].  A call that cuts the input columns
    into workgroup chunks needs a workspace whose counters are zero; without
    `ws` the stream's cached one is used."""
    import torch
    M = qx.shape[0]
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=qx.device)
    need = aq_workspace_bytes(pw, M, AQ_PHASE_DECODE, split)
    if ws is None and need:
        ws = decode_workspace(need, qx.device, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().aq_linear_decode(ctypes.byref(pw.desc), _ptr(qx), _ptr(sx), M, _ptr(bias),
                                  _ptr(out), split, _ptr(ws), ws_bytes, _stream(stream)),
           "aq_linear_decode")
    return out


def aq_linear_decode_fp32(pw: PackedWeights, X, bias=None, split: int = 0, out=None, ws=None,
                          stream=None):
    """Decode-phase linear from FP32 activations X [M, K]: the per-token
    quantization and the linear in one call (one kernel for up to 4 tokens
    with M*K <= 8192); FP32 Y [M, N], bit for bit aq_quant_act followed by
    aq_linear_decode.  Without `ws` the stream's cached decode workspace is
    used when the call needs one."""
    import torch
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=X.device)
    need = aq_workspace_bytes(pw, M, AQ_PHASE_DECODE_FP32, split)
    if ws is None and need:
        ws = decode_workspace(need, X.device, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().aq_linear_decode_fp32(ctypes.byref(pw.desc), _ptr(X), M, _ptr(bias), _ptr(out), split,
                                       _ptr(ws), ws_bytes, _stream(stream)),
           "aq_linear_decode_fp32")
    return out


AQ_DECODE_SCRATCH_BYTES = 8 << 20


def aq_linear_decode_noalloc(pw: PackedWeights, qx, sx, out, bias=None, split: int = 0, stream=None):
    """aq_linear_decode with the library's own device scratch in place of a
    workspace: the C call allocates nothing; the caller provides `out`
    (FP32 [M, N])."""
    M = qx.shape[0]
    _check(lib().aq_linear_decode_noalloc(ctypes.byref(pw.desc), _ptr(qx), _ptr(sx), M, _ptr(bias),
                                          _ptr(out), split, _stream(stream)),
           "aq_linear_decode_noalloc")
    return out


def _workspace(pw: PackedWeights, M: int, phase: int, ws, device):
    import torch
    need = aq_workspace_bytes(pw, M, phase, 0)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def aq_linear_prefill(pw: PackedWeights, qx, sx, bias=None, out=None, ws=None, stream=None):
    """Prefill-phase linear (INT8 MFMA): FP32 Y [M, N].  A long prompt on a
    projection with INT4 tiles needs a workspace (allocated here if not given)."""
    import torch
    M = qx.shape[0]
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=qx.device)
    ws, ws_bytes = _workspace(pw, M, AQ_PHASE_PREFILL, ws, qx.device)
    _check(lib().aq_linear_prefill(ctypes.byref(pw.desc), _ptr(qx), _ptr(sx), M, _ptr(bias),
                                   _ptr(out), _ptr(ws), ws_bytes, _stream(stream)), "aq_linear_prefill")
    return out


def aq_prefill_prepare(pw: PackedWeights, ws, stream=None):
    """Write the long-prompt temporary INT8 operand of pw into ws (a device
    uint8 tensor of at least aq_workspace_bytes(pw, 1024, prefill) bytes);
    a no-op when the projection needs none."""
    need = aq_workspace_bytes(pw, 1024, AQ_PHASE_PREFILL)
    _check(lib().aq_prefill_prepare(ctypes.byref(pw.desc), _ptr(ws) if need else None,
                                    ws.numel() * ws.element_size() if (need and ws is not None) else 0, _stream(stream)),
           "aq_prefill_prepare")


def aq_linear_prefill_prepared(pw: PackedWeights, qx, sx, ws, bias=None, out=None, stream=None):
    """aq_linear_prefill over an operand aq_prefill_prepare already wrote to ws."""
    import torch
    M = qx.shape[0]
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=qx.device)
    need = aq_workspace_bytes(pw, M, AQ_PHASE_PREFILL)
    _check(lib().aq_linear_prefill_prepared(ctypes.byref(pw.desc), _ptr(qx), _ptr(sx), M, _ptr(bias), _ptr(out),
                                            _ptr(ws) if need else None,
                                            ws.numel() * ws.element_size() if (need and ws is not None) else 0, _stream(stream)),
           "aq_linear_prefill_prepared")
    return out


def aq_linear_tile_partials(pw: PackedWeights, qx, phase: int, out=None, ws=None, stream=None):
    """INT32 tile products P [M, N, C] computed by the decode or prefill kernels."""
    import torch
    M = qx.shape[0]
    C = pw.plan.C
    if out is None:
        out = torch.empty((M, pw.N, C), dtype=torch.int32, device=qx.device)
    ws, ws_bytes = (None, 0) if phase != AQ_PHASE_PREFILL else _workspace(pw, M, phase, ws, qx.device)
    _check(lib().aq_linear_tile_partials(ctypes.byref(pw.desc), _ptr(qx), M, phase, _ptr(out),
                                         _ptr(ws), ws_bytes, _stream(stream)), "aq_linear_tile_partials")
    return out


# ---------------------------------------------------------------- App. B.3 activation groups

def aq_act_group_shape(M: int, K: int) -> tuple[int, int, int]:
    """(b_M, rows, cols) of the App. B.3 activation-scale array for M rows of
    K features, as the library defines them (host only)."""
    bM, rows, cols = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().aq_act_group_shape(M, K, ctypes.byref(bM), ctypes.byref(rows), ctypes.byref(cols)),
           "aq_act_group_shape")
    return bM.value, rows.value, cols.value


def aq_quant_act_grouped(X, qx=None, sxg=None, stream=None):
    """INT8 codes [M, K] and FP32 group scales [rows, cols] of device FP32
    X [M, K], shaped by aq_act_group_shape (one scale per 64 features x b_M
    rows, eq. 6)."""
    import torch
    M, K = X.shape
    _, G, KG = aq_act_group_shape(M, K)
    if qx is None:
        qx = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if sxg is None:
        sxg = torch.empty((G, KG), dtype=torch.float32, device=X.device)
    _check(lib().aq_quant_act_grouped(ctypes.c_void_p(X.data_ptr()), M, K, ctypes.c_void_p(qx.data_ptr()),
                                      ctypes.c_void_p(sxg.data_ptr()), _stream(stream)),
           "aq_quant_act_grouped")
    return qx, sxg


def aq_linear_decode_grouped(pw: PackedWeights, qx, sxg, bias=None, split: int = 0, out=None, ws=None,
                             stream=None):
    """Decode-phase linear with App. B.3 group scales: FP32 Y [M, N]."""
    import torch
    M = qx.shape[0]
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=qx.device)
    need = aq_workspace_bytes(pw, M, AQ_PHASE_DECODE, split)
    if ws is None and need:
        ws = decode_workspace(need, qx.device, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().aq_linear_decode_grouped(ctypes.byref(pw.desc), _ptr(qx), _ptr(sxg), M, _ptr(bias),
                                          _ptr(out), split, _ptr(ws), ws_bytes, _stream(stream)),
           "aq_linear_decode_grouped")
    return out


def _grouped_workspace(pw: PackedWeights, M: int, ws, device, stream=None):
    """The workspace of the grouped prefill for M rows: the library sizes it;
    a workspace as large as the long-prompt one belongs to the long route
    (the temporary operand), any other to the decode kernels (the stream's
    zeroed decode workspace, whose counters must stay apart from operands)."""
    import torch
    need = aq_workspace_bytes(pw, M, AQ_PHASE_PREFILL_GROUPED)
    if ws is None and need:
        if aq_workspace_bytes(pw, M, AQ_PHASE_PREFILL) == need:
            ws = torch.empty(need, dtype=torch.uint8, device=device)
        else:
            ws = decode_workspace(need, device, stream)
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def aq_linear_prefill_grouped(pw: PackedWeights, qx, sxg, bias=None, out=None, ws=None, stream=None):
    """Any-length linear with App. B.3 group scales: the long-prompt GEMM for
    long prompts, else the decode kernels."""
    import torch
    M = qx.shape[0]
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=qx.device)
    ws, ws_bytes = _grouped_workspace(pw, M, ws, qx.device, stream)
    _check(lib().aq_linear_prefill_grouped(ctypes.byref(pw.desc), _ptr(qx), _ptr(sxg), M, _ptr(bias),
                                           _ptr(out), _ptr(ws), ws_bytes, _stream(stream)),
           "aq_linear_prefill_grouped")
    return out


def aq_linear_tile_partials_grouped(pw: PackedWeights, qx, out=None, ws=None, stream=None):
    """INT32 group products P [M, N, K/64] of the grouped eq. 19, from the
    kernels aq_linear_prefill_grouped takes for M rows."""
    import torch
    M = qx.shape[0]
    if out is None:
        out = torch.empty((M, pw.N, pw.K // 64), dtype=torch.int32, device=qx.device)
    ws, ws_bytes = _grouped_workspace(pw, M, ws, qx.device, stream)
    _check(lib().aq_linear_tile_partials_grouped(ctypes.byref(pw.desc), _ptr(qx), M, _ptr(out), _ptr(ws),
                                                 ws_bytes, _stream(stream)), "aq_linear_tile_partials_grouped")
    return out


# ------------------------------------------------ block transforms (App. B.1)

def transform_tables(perm, dl, dr) -> AqTransformTables:
    """The six signed permutations (perm uint8 [6, 64], dl / dr int8 [6, 64]
    of +-1) as the C struct the transform calls read."""
    t = AqTransformTables()
    perm = np.ascontiguousarray(perm, dtype=np.uint8).reshape(6, 64)
    dl = np.ascontiguousarray(dl, dtype=np.int8).reshape(6, 64)
    dr = np.ascontiguousarray(dr, dtype=np.int8).reshape(6, 64)
    ctypes.memmove(ctypes.addressof(t.perm), perm.ctypes.data, perm.nbytes)
    ctypes.memmove(ctypes.addressof(t.dl), dl.ctypes.data, dl.nbytes)
    ctypes.memmove(ctypes.addressof(t.dr), dr.ctypes.data, dr.nbytes)
    return t


def _seeds_dev(seeds, n: int, device):
    """The n block seeds as a device INT8 tensor (the C calls read n)."""
    import torch
    if isinstance(seeds, torch.Tensor):
        if not (seeds.dtype == torch.int8 and seeds.is_contiguous() and seeds.device.type == "cuda"):
            raise ValueError("seeds must be a contiguous int8 device tensor")
    else:
        seeds = torch.as_tensor(np.asarray(seeds, dtype=np.int8)).to(device)
    if seeds.numel() != n:
        raise ValueError(f"expected {n} block seeds, got {seeds.numel()}")
    return seeds


def _check_f32(t, shape, what):
    import torch
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must be a contiguous float32 tensor of shape {tuple(shape)}")


def _tables(tables) -> AqTransformTables:
    return tables if isinstance(tables, AqTransformTables) else transform_tables(*tables)


def aq_transform_rows(X, vseeds, tables, out=None, stream=None):
    """X~ = X V (FP32 [M, K] on the device); vseeds: K/64 seeds in -1..6."""
    import torch
    M, K = X.shape
    if out is None:
        out = torch.empty_like(X)
    _check_f32(X, (M, K), "X")
    _check_f32(out, (M, K), "out")
    sd = _seeds_dev(vseeds, K // 64, X.device)
    t = _tables(tables)
    _check(lib().aq_transform_rows(ctypes.c_void_p(X.data_ptr()), M, K, ctypes.c_void_p(sd.data_ptr()),
                                   ctypes.byref(t), ctypes.c_void_p(out.data_ptr()), _stream(stream)),
           "aq_transform_rows")
    return out


def aq_transform_out(Yt, useeds, tables, bias=None, out=None, stream=None):
    """Y = Y~ U + bias (FP32 [M, N] on the device; out=Yt transforms in place)."""
    import torch
    M, N = Yt.shape
    if out is None:
        out = torch.empty_like(Yt)
    _check_f32(Yt, (M, N), "Yt")
    _check_f32(out, (M, N), "out")
    if bias is not None:
        _check_f32(bias, (N,), "bias")
    sd = _seeds_dev(useeds, N // 64, Yt.device)
    t = _tables(tables)
    _check(lib().aq_transform_out(ctypes.c_void_p(Yt.data_ptr()), M, N, ctypes.c_void_p(sd.data_ptr()),
                                  ctypes.byref(t), _ptr(bias), ctypes.c_void_p(out.data_ptr()),
                                  _stream(stream)),
           "aq_transform_out")
    return out


def aq_quant_act_transformed(X, vseeds, tables, qx=None, sx=None, stream=None):
    """INT8 codes [M, K] and FP32 per-token scales [M] of X~ = X V, computed
    in one pass (X FP32 [M, K] on the device, K <= 40768)."""
    import torch
    M, K = X.shape
    _check_f32(X, (M, K), "X")
    if qx is None:
        qx = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if sx is None:
        sx = torch.empty((M,), dtype=torch.float32, device=X.device)
    sd = _seeds_dev(vseeds, K // 64, X.device)
    t = _tables(tables)
    _check(lib().aq_quant_act_transformed(ctypes.c_void_p(X.data_ptr()), M, K, ctypes.c_void_p(sd.data_ptr()),
                                          ctypes.byref(t), ctypes.c_void_p(qx.data_ptr()),
                                          ctypes.c_void_p(sx.data_ptr()), _stream(stream)),
           "aq_quant_act_transformed")
    return qx, sx


def aq_transform_weights(W, useeds, vseeds, tables, out=None, stream=None):
    """W~ = U W V (FP32 [N, K] on the device)."""
    import torch
    N, K = W.shape
    if out is None:
        out = torch.empty_like(W)
    _check_f32(W, (N, K), "W")
    _check_f32(out, (N, K), "out")
    su = _seeds_dev(useeds, N // 64, W.device)
    sv = _seeds_dev(vseeds, K // 64, W.device)
    t = _tables(tables)
    _check(lib().aq_transform_weights(ctypes.c_void_p(W.data_ptr()), N, K, ctypes.c_void_p(su.data_ptr()),
                                      ctypes.c_void_p(sv.data_ptr()), ctypes.byref(t),
                                      ctypes.c_void_p(out.data_ptr()), _stream(stream)),
           "aq_transform_weights")
    return out


def aq_linear_decode_transformed(pw: PackedWeights, qx, sx, useeds, tables, bias=None, split: int = 0,
                                 out=None, ws=None, stream=None):
    """Y = Y~ U + bias for a transformed layer's decode call, U applied in
    the decode epilogue: FP32 [M, N].  Without `ws` the stream's cached
    decode workspace is used."""
    import torch
    M = qx.shape[0]
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=qx.device)
    need = aq_workspace_bytes(pw, M, AQ_PHASE_DECODE_TRANSFORMED, split)
    if ws is None and need:
        ws = decode_workspace(need, qx.device, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    sd = _seeds_dev(useeds, pw.N // 64, qx.device)
    t = _tables(tables)
    _check(lib().aq_linear_decode_transformed(ctypes.byref(pw.desc), _ptr(qx), _ptr(sx), M, _ptr(bias),
                                              ctypes.c_void_p(sd.data_ptr()), ctypes.byref(t), _ptr(out),
                                              split, _ptr(ws), ws_bytes, _stream(stream)),
           "aq_linear_decode_transformed")
    return out


def aq_linear_prefill_transformed(pw: PackedWeights, qx, sx, useeds, tables, bias=None, out=None, ws=None,
                                  stream=None):
    """Y = Y~ U + bias for a transformed layer (long prompts apply U inside
    the GEMM): FP32 [M, N]."""
    import torch
    M = qx.shape[0]
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=qx.device)
    ws, ws_bytes = _workspace(pw, M, AQ_PHASE_PREFILL, ws, qx.device)
    sd = _seeds_dev(useeds, pw.N // 64, qx.device)
    t = _tables(tables)
    _check(lib().aq_linear_prefill_transformed(ctypes.byref(pw.desc), _ptr(qx), _ptr(sx), M, _ptr(bias),
                                               ctypes.c_void_p(sd.data_ptr()), ctypes.byref(t), _ptr(out),
                                               _ptr(ws), ws_bytes, _stream(stream)),
           "aq_linear_prefill_transformed")
    return out
