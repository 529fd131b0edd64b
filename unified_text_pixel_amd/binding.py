"""ctypes binding of libha.so: the C-ABI entry points under the same names.

Argument marshalling only: tensors become device pointers, the stream becomes the
caller's current HIP stream, a nonzero status raises HAError. Every step of the path runs
in the HIP kernels of libha.so; there is no fallback of any kind. PyTorch supplies device
memory and streams (torch is imported before the library so both share one HIP runtime).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libha.so")

HA_OK, HA_ERR_INVALID_ARG, HA_ERR_UNSUPPORTED, HA_ERR_SEGMENTS = 0, 1, 2, 3
HA_ERR_ALIGNMENT, HA_ERR_WORKSPACE, HA_ERR_HIP = 4, 5, 6
HA_SEG_CAUSAL, HA_SEG_FULL, HA_SEG_GCA, HA_SEG_GEN = 0, 1, 2, 3
HA_DTYPE_BF16, HA_DTYPE_F32 = 0, 1
HA_ROPE_NONE, HA_ROPE_1D, HA_ROPE_2D, HA_ROPE_MROPE = 0, 1, 2, 3
HA_TILE_SKIP, HA_TILE_FULL, HA_TILE_PARTIAL = 0, 1, 2
ROPE_KINDS = {"none": HA_ROPE_NONE, "1d": HA_ROPE_1D, "2d": HA_ROPE_2D, "mrope": HA_ROPE_MROPE}

# Every function include/ha_attn.h declares.
EXPORTS = ("ha_abi_version", "ha_last_error", "ha_rope_table_fill", "ha_q_prescale",
           "ha_tile_shape", "ha_classify_tiles", "ha_qk_prologue", "ha_attn_workspace_bytes",
           "ha_attn_fwd_planned", "ha_attn_fwd", "ha_attn_fwd_lse", "ha_attn_bwd_workspace_bytes",
           "ha_attn_bwd", "ha_qk_prologue_from", "ha_attn_fwd_planned_from", "ha_qkv_prologue",
           "ha_attn_fwd_static")


class HAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"ha status {status}: {message}")
        self.status = status


class ha_segment(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int32), ("length", ctypes.c_int32), ("kind", ctypes.c_int32)]


class ha_attn_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("segments", ctypes.POINTER(ha_segment)), ("n_segments", ctypes.c_int32),
                ("scale", ctypes.c_float), ("q_prescaled", ctypes.c_int32),
                ("split_parts", ctypes.c_int32), ("plan_cus", ctypes.c_int32)]


class ha_prologue_desc(ctypes.Structure):
    _fields_ = [("rope_kind", ctypes.c_int32), ("mrope_sections", ctypes.c_int32 * 3),
                ("positions", ctypes.c_void_p), ("cos_sin", ctypes.c_void_p),
                ("n_pos", ctypes.c_int32), ("q_norm_weight", ctypes.c_void_p),
                ("k_norm_weight", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("q_out_scale", ctypes.c_float)]


_lib = None


def load_library(path: str = LIB_PATH, with_torch: bool = True):
    """Load libha.so once. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m unified_text_pixel_amd.build)")
    if with_torch:
        import torch  # noqa: F401  (shares its HIP runtime with the library)
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D, PD = ctypes.POINTER(ha_attn_desc), ctypes.POINTER(ha_prologue_desc)
    sig = {
        "ha_abi_version": ([], ctypes.c_int),
        "ha_last_error": ([], ctypes.c_char_p),
        "ha_rope_table_fill": ([ctypes.c_double, I32, I32, P], ctypes.c_int),
        "ha_q_prescale": ([D], ctypes.c_float),
        "ha_tile_shape": ([D, P, P, P, P], ctypes.c_int),
        "ha_classify_tiles": ([D, P, P, P, P], ctypes.c_int),
        "ha_qk_prologue": ([D, PD, P, P, P, P, P], ctypes.c_int),
        "ha_attn_workspace_bytes": ([D, PD], SZ),
        "ha_attn_fwd_planned": ([D, P, P, P, P, P, P, P], ctypes.c_int),
        "ha_attn_fwd": ([D, PD, P, P, P, P, P, SZ, P], ctypes.c_int),
        "ha_attn_fwd_lse": ([D, PD, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "ha_attn_bwd_workspace_bytes": ([D, PD], SZ),
        "ha_attn_bwd": ([D, PD, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "ha_qk_prologue_from": ([D, PD, P, P, P, P, I32, P], ctypes.c_int),
        "ha_attn_fwd_planned_from": ([D, P, P, P, P, P, P, I32, P], ctypes.c_int),
        "ha_qkv_prologue": ([D, PD, P, I32, P, P, P, P, P], ctypes.c_int),
        "ha_attn_fwd_static": ([D, P, P, P, P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int):
    if status != HA_OK:
        raise HAError(status, _lib.ha_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class AttnDesc:
    """Owns an ha_attn_desc and the host segment array it points to."""

    def __init__(self, batch, seq_len, n_q_heads, n_kv_heads, head_dim, dtype, segments,
                 scale: float = 0.0, q_prescaled: int = 0, split_parts: int = 0, plan_cus: int = 0):
        seg = np.asarray(segments, dtype=np.int32)
        if batch > 0 and seq_len > 0:
            seg = np.ascontiguousarray(seg.reshape(batch, -1, 3))
        else:
            seg = np.zeros((0, 0, 3), np.int32)
        self._seg_np = seg
        n_seg = seg.shape[1] if seg.size else 0
        self._seg = (ha_segment * max(1, seg.shape[0] * n_seg))()
        for idx, (st, ln, kd) in enumerate(seg.reshape(-1, 3)):
            self._seg[idx] = ha_segment(int(st), int(ln), int(kd))
        dt = {"bf16": HA_DTYPE_BF16, "f32": HA_DTYPE_F32}.get(dtype, dtype)
        self.c = ha_attn_desc(batch, seq_len, n_q_heads, n_kv_heads, head_dim, dt,
                              ctypes.cast(self._seg, ctypes.POINTER(ha_segment)), n_seg,
                              float(scale), int(q_prescaled), int(split_parts), int(plan_cus))


class PrologueDesc:
    def __init__(self, rope_kind, positions=None, cos_sin=None, n_pos=0, q_norm_weight=None,
                 k_norm_weight=None, eps=1e-6, mrope_sections=(0, 0, 0), q_out_scale=0.0):
        kind = ROPE_KINDS.get(rope_kind, rope_kind)
        self._keep = (positions, cos_sin, q_norm_weight, k_norm_weight)
        self.c = ha_prologue_desc(kind, (ctypes.c_int32 * 3)(*mrope_sections), _ptr(positions),
                                  _ptr(cos_sin), int(n_pos), _ptr(q_norm_weight),
                                  _ptr(k_norm_weight), float(eps), float(q_out_scale))


def _d(desc):
    return ctypes.byref(desc.c)


def _pd(pro):
    return None if pro is None else ctypes.byref(pro.c)


# ---------------------------------------------------------------- the C-ABI entry points
def ha_abi_version() -> int:
    return load_library().ha_abi_version()


def ha_last_error() -> str:
    return load_library().ha_last_error().decode()


def ha_rope_table_fill(theta: float, head_dim: int, n_pos: int) -> np.ndarray:
    """Host (cos, sin) table float32 [n_pos][head_dim/2][2]."""
    lib = load_library()
    out = np.empty((max(n_pos, 0), head_dim // 2, 2), dtype=np.float32)
    _check(lib.ha_rope_table_fill(float(theta), head_dim, n_pos,
                                  out.ctypes.data_as(ctypes.c_void_p) if out.size else None))
    return out


def ha_q_prescale(desc: AttnDesc) -> float:
    """scale * log2(e): the factor a prescaled q carries (0.0 for an invalid descriptor)."""
    return float(load_library().ha_q_prescale(_d(desc)))


def ha_tile_shape(desc: AttnDesc):
    lib = load_library()
    v = [ctypes.c_int32() for _ in range(4)]
    _check(lib.ha_tile_shape(_d(desc), *[ctypes.byref(x) for x in v]))
    return tuple(x.value for x in v)  # block_q, block_k, n_q_blocks, n_k_blocks


def ha_classify_tiles(desc: AttnDesc, labels=None, ranges=None, row_limit=None, stream=None):
    _check(load_library().ha_classify_tiles(_d(desc), _ptr(labels), _ptr(ranges),
                                            _ptr(row_limit), _stream(stream)))


def ha_qk_prologue(desc: AttnDesc, pro: PrologueDesc, q_in, k_in, q_out, k_out, stream=None):
    _check(load_library().ha_qk_prologue(_d(desc), _pd(pro), _ptr(q_in), _ptr(k_in),
                                         _ptr(q_out), _ptr(k_out), _stream(stream)))


def ha_attn_workspace_bytes(desc: AttnDesc, pro: Optional[PrologueDesc] = None) -> int:
    return load_library().ha_attn_workspace_bytes(_d(desc), _pd(pro))


def ha_attn_fwd_planned(desc: AttnDesc, q, k, v, row_limit, ranges, out, stream=None):
    _check(load_library().ha_attn_fwd_planned(_d(desc), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(row_limit), _ptr(ranges), _ptr(out),
                                              _stream(stream)))


def ha_attn_fwd(desc: AttnDesc, pro: Optional[PrologueDesc], q, k, v, out, workspace,
                workspace_bytes: Optional[int] = None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().ha_attn_fwd(_d(desc), _pd(pro), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                      _ptr(workspace), int(workspace_bytes), _stream(stream)))


def _nbytes(workspace, workspace_bytes):
    if workspace_bytes is not None:
        return int(workspace_bytes)
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def ha_attn_fwd_lse(desc: AttnDesc, pro: Optional[PrologueDesc], q, k, v, out, lse, workspace,
                    workspace_bytes: Optional[int] = None, stream=None):
    _check(load_library().ha_attn_fwd_lse(_d(desc), _pd(pro), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                          _ptr(lse), _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                          _stream(stream)))


def ha_attn_bwd_workspace_bytes(desc: AttnDesc, pro: Optional[PrologueDesc] = None) -> int:
    return load_library().ha_attn_bwd_workspace_bytes(_d(desc), _pd(pro))


def ha_attn_bwd(desc: AttnDesc, pro: Optional[PrologueDesc], q, k, v, out, lse, dout, dq, dk, dv,
                dw_q, dw_k, workspace, workspace_bytes: Optional[int] = None, stream=None):
    _check(load_library().ha_attn_bwd(_d(desc), _pd(pro), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                      _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dw_q),
                                      _ptr(dw_k), _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                      _stream(stream)))


def ha_qk_prologue_from(desc: AttnDesc, pro: PrologueDesc, q_in, k_in, q_out, k_out, token_begin: int,
                        stream=None):
    _check(load_library().ha_qk_prologue_from(_d(desc), _pd(pro), _ptr(q_in), _ptr(k_in), _ptr(q_out),
                                              _ptr(k_out), int(token_begin), _stream(stream)))


def ha_attn_fwd_planned_from(desc: AttnDesc, q, k, v, row_limit, ranges, out, row_begin: int, stream=None):
    _check(load_library().ha_attn_fwd_planned_from(_d(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(row_limit),
                                                   _ptr(ranges), _ptr(out), int(row_begin), _stream(stream)))


def ha_qkv_prologue(desc: AttnDesc, pro, x, hidden: int, w_qkv, q_out, k_out, v_out, stream=None):
    _check(load_library().ha_qkv_prologue(_d(desc), _pd(pro), _ptr(x), int(hidden), _ptr(w_qkv), _ptr(q_out),
                                          _ptr(k_out), _ptr(v_out), _stream(stream)))


def ha_attn_fwd_static(desc: AttnDesc, q, k, v, out, stream=None):
    _check(load_library().ha_attn_fwd_static(_d(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _stream(stream)))
