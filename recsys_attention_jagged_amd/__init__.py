"""Python binding of libgdpa, the MI355X jagged GDPA library (argument marshalling only).

Every function mirrors the C entry point of the same name in include/gdpa.h;
tensors may be passed as torch tensors (their data pointers are used) or as
raw integer addresses.  All GDPA arithmetic runs in the library's HIP kernels;
PyTorch is used here only to hand over device memory and streams.  If the
library has not been built, loading it raises: there is no fallback.

Build it with ``python -m recsys_attention_jagged_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdpa.so")

GDPA_OK = 0
STATUS = {0: "GDPA_OK", 1: "GDPA_ERR_INVALID_ARG", 2: "GDPA_ERR_BAD_OFFSETS", 3: "GDPA_ERR_UNSUPPORTED",
          4: "GDPA_ERR_PLAN_MISMATCH", 5: "GDPA_ERR_HIP", 6: "GDPA_ERR_NOMEM"}
ACT = {"gelu": 0, "silu": 1, "gelu_poly": 2, "gelu_taylor6": 3, "identity": 4, "one": 5}
DTYPE = {"f32": 0, "bf16": 1, "bf16_f32out": 2}
LIST = {"fwd": 0, "dkdv": 1, "dq": 2, "dq_team": 3}
DEAL = {"greedy": 0, "zigzag": 1, "round_robin": 2}


class GdpaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class gdpa_plan_opts(ctypes.Structure):
    _fields_ = [("host_only", ctypes.c_int), ("bins", ctypes.c_int * 3), ("team", ctypes.c_int * 3),
                ("blocks", ctypes.c_int * 3), ("deal", ctypes.c_int), ("no_split", ctypes.c_int),
                ("unfused", ctypes.c_int), ("no_ds", ctypes.c_int), ("claim", ctypes.c_int),
                ("slot_time", ctypes.c_int), ("dq_team", ctypes.c_int)]


class gdpa_plan_stats_t(ctypes.Structure):
    _fields_ = [("Tq", ctypes.c_int64), ("Tk", ctypes.c_int64), ("valid_pairs", ctypes.c_int64),
                ("n_items", ctypes.c_int32 * 3), ("n_steps", ctypes.c_int32 * 3),
                ("bins", ctypes.c_int32 * 3), ("tile_stat", ctypes.c_int32 * 3),
                ("tile_strm", ctypes.c_int32 * 3), ("bin_cost_max", ctypes.c_int64 * 3),
                ("bin_cost_min", ctypes.c_int64 * 3), ("bwd_fused", ctypes.c_int32),
                ("n_parts", ctypes.c_int32 * 3), ("ds_bytes", ctypes.c_int64), ("claimed", ctypes.c_int32 * 3),
                ("slot_weighted", ctypes.c_int32 * 3), ("dq_team", ctypes.c_int32),
                ("dq_team_items", ctypes.c_int32), ("dq_team_bins", ctypes.c_int32), ("dq_team_parts", ctypes.c_int32),
                ("dq_team_slot_weighted", ctypes.c_int32)]


_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libgdpa.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run: python -m recsys_attention_jagged_amd.build")
    lib = ctypes.CDLL(path)
    lib.gdpa_plan_create.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, ctypes.POINTER(gdpa_plan_opts), _vp,
                                     ctypes.POINTER(_vp)]
    lib.gdpa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]
    lib.gdpa_fwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]
    lib.gdpa_mx_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]
    lib.gdpa_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp]
    lib.gdpa_bwd_dkdv.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp]
    lib.gdpa_bwd_dq.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]
    lib.gdpa_plan_export.argtypes = [_vp, _i, _vp, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdpa_plan_stats.argtypes = [_vp, ctypes.POINTER(gdpa_plan_stats_t)]
    lib.gdpa_plan_destroy.argtypes = [_vp]
    lib.gdpa_plan_destroy.restype = None
    lib.gdpa_status_string.argtypes = [_i]
    lib.gdpa_status_string.restype = ctypes.c_char_p
    lib.gdpa_last_error.argtypes = []
    lib.gdpa_last_error.restype = ctypes.c_char_p
    lib.gdpa_gelu_poly_bound.argtypes = []
    lib.gdpa_gelu_poly_bound.restype = ctypes.c_double
    lib.gdpa_gelu_poly_grad_bound.argtypes = []
    lib.gdpa_gelu_poly_grad_bound.restype = ctypes.c_double
    lib.gdpa_jfa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp]
    lib.gdpa_jfa_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp,
                                 _vp]
    lib.gdpa_fp8_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, ctypes.c_float, ctypes.c_float,
                                 _vp, _vp]
    lib.gdpa_fp8_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, ctypes.c_float,
                                 ctypes.c_float, ctypes.c_float, _vp, _vp, _vp, _vp]
    lib.gdpa_norm_rstd.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp]
    lib.gdpa_norm_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]
    lib.gdpa_norm_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp,
                                  _vp]
    lib.gdpa_norm_bwd_dkdv.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp,
                                       _vp]
    lib.gdpa_norm_bwd_dq.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]
    lib.gdpa_jfa_bwd_stat.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _vp, _vp]
    lib.gdpa_jfa_bwd_dkdv.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp]
    lib.gdpa_jfa_bwd_dq.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp]
    lib.gdpa_pffn_plan_create.argtypes = [_i, _i, _i, _i, _i, ctypes.POINTER(gdpa_plan_opts), _vp,
                                          ctypes.POINTER(_vp)]
    lib.gdpa_pffn_fwd.argtypes = [_vp, _vp, _vp, _vp, _i, _vp, _vp]
    lib.gdpa_pffn_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp]
    for name in ("gdpa_plan_create", "gdpa_fwd", "gdpa_fwd_noalloc", "gdpa_bwd", "gdpa_bwd_dkdv", "gdpa_bwd_dq",
                 "gdpa_plan_export", "gdpa_plan_stats", "gdpa_pffn_plan_create", "gdpa_pffn_fwd",
                 "gdpa_pffn_bwd", "gdpa_jfa_fwd", "gdpa_jfa_bwd", "gdpa_jfa_bwd_stat", "gdpa_jfa_bwd_dkdv",
                 "gdpa_jfa_bwd_dq", "gdpa_norm_rstd", "gdpa_norm_fwd", "gdpa_norm_bwd", "gdpa_norm_bwd_dkdv",
                 "gdpa_norm_bwd_dq", "gdpa_fp8_fwd", "gdpa_fp8_bwd", "gdpa_mx_fwd"):
        getattr(lib, name).restype = _i
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status: int):
    if status != GDPA_OK:
        raise GdpaError(status, load_library().gdpa_last_error().decode())


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr() or None
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _enum(v, table):
    return table[v] if isinstance(v, str) else int(v)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def gdpa_plan_create(q_off_host, kv_off_host, B: int, H: int, d: int, window: int, dtype,
                     host_only: bool = False, bins=(0, 0, 0), team=(0, 0, 0), blocks=(0, 0, 0),
                     deal="greedy", split: bool = True, unfused: bool = False, stream=None,
                     store_ds: bool = True, claim="auto", slot_time="auto", dq_team="auto") -> int:
    """Returns an opaque plan handle (int).  Offsets: host int32 [B + 1].  The work
    lists are copied on `stream` (torch's current stream by default; none for a
    host-only plan)."""
    qo = np.ascontiguousarray(q_off_host, dtype=np.int32)
    ko = np.ascontiguousarray(kv_off_host, dtype=np.int32)
    if qo.shape != (B + 1,) or ko.shape != (B + 1,):
        raise ValueError("offsets must have B + 1 entries")
    opts = _opts(host_only, bins, team, blocks, deal, split, unfused, store_ds, claim, slot_time, dq_team)
    out = _vp()
    _check(load_library().gdpa_plan_create(qo.ctypes.data, ko.ctypes.data, B, H, d, window,
                                           _enum(dtype, DTYPE), ctypes.byref(opts),
                                           None if host_only else _stream(stream), ctypes.byref(out)))
    return out.value


def gdpa_fwd(plan, q, k, v, q_off_dev, kv_off_dev, B, H, d, act, window, o, stream=None):
    _check(load_library().gdpa_fwd(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(q_off_dev), _ptr(kv_off_dev),
                                   B, H, d, _enum(act, ACT), window, _ptr(o), _stream(stream)))


def gdpa_fwd_noalloc(plan, q, k, v, q_off_dev, kv_off_dev, B, H, d, act, window, o, stream=None):
    """gdpa_fwd without any allocation: the work list goes into the library's fixed scratch array."""
    _check(load_library().gdpa_fwd_noalloc(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(q_off_dev), _ptr(kv_off_dev),
                                           B, H, d, _enum(act, ACT), window, _ptr(o), _stream(stream)))


def gdpa_bwd(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, act, window, dq, dk, dv,
             stream=None):
    _check(load_library().gdpa_bwd(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(q_off_dev),
                                   _ptr(kv_off_dev), B, H, d, _enum(act, ACT), window, _ptr(dq),
                                   _ptr(dk), _ptr(dv), _stream(stream)))


def gdpa_bwd_dkdv(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, act, window, dk, dv, stream=None):
    _check(load_library().gdpa_bwd_dkdv(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(q_off_dev),
                                        _ptr(kv_off_dev), B, H, d, _enum(act, ACT), window, _ptr(dk),
                                        _ptr(dv), _stream(stream)))


def gdpa_bwd_dq(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, act, window, dq, stream=None):
    _check(load_library().gdpa_bwd_dq(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(q_off_dev),
                                      _ptr(kv_off_dev), B, H, d, _enum(act, ACT), window, _ptr(dq),
                                      _stream(stream)))


def gdpa_jfa_fwd(plan, q, k, v, q_off_dev, kv_off_dev, B, H, d, window, o, lse, stream=None):
    """Jagged softmax attention: O [Tq, H, d] and LSE fp32 [H, Tq]."""
    _check(load_library().gdpa_jfa_fwd(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(q_off_dev), _ptr(kv_off_dev),
                                       B, H, d, window, _ptr(o), _ptr(lse), _stream(stream)))


def gdpa_jfa_bwd(plan, q, k, v, o, lse, dout, q_off_dev, kv_off_dev, B, H, d, window, stat, dq, dk, dv,
                 stream=None):
    """Gradients of jagged softmax attention from its O and LSE; stat is fp32 [H, Tq, 2] scratch."""
    _check(load_library().gdpa_jfa_bwd(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                       _ptr(q_off_dev), _ptr(kv_off_dev), B, H, d, window, _ptr(stat), _ptr(dq),
                                       _ptr(dk), _ptr(dv), _stream(stream)))


def gdpa_jfa_bwd_stat(plan, o, lse, dout, H, d, stat, stream=None):
    """The JFA backward's pre-pass: stat [H, Tq, 2] = (LSE log2 e, sum dO * O)."""
    _check(load_library().gdpa_jfa_bwd_stat(plan, _ptr(o), _ptr(lse), _ptr(dout), H, d, _ptr(stat),
                                            _stream(stream)))


def gdpa_jfa_bwd_dkdv(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, window, stat, dk, dv, stream=None):
    _check(load_library().gdpa_jfa_bwd_dkdv(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(q_off_dev),
                                            _ptr(kv_off_dev), B, H, d, window, _ptr(stat), _ptr(dk), _ptr(dv),
                                            _stream(stream)))


def gdpa_jfa_bwd_dq(plan, q, k, v, o, lse, dout, q_off_dev, kv_off_dev, B, H, d, window, stat, dq, stream=None):
    """dQ of the JFA backward; also writes stat (LSE log2 e, D) for gdpa_jfa_bwd_dkdv."""
    _check(load_library().gdpa_jfa_bwd_dq(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                          _ptr(q_off_dev), _ptr(kv_off_dev), B, H, d, window, _ptr(stat), _ptr(dq),
                                          _stream(stream)))


NORM_BITS = {"q": 1, "k": 2, "v": 4}


def norm_code(norm) -> int:
    """"qkv"-style subset (or an int 0..7) -> the library's norm bits."""
    if isinstance(norm, int):
        return norm
    return sum(NORM_BITS[c] for c in set(norm))


def gdpa_fp8_fwd(plan, q8, k8, v, q_off_dev, kv_off_dev, B, H, d, act, window, q_scale, k_scale, o, stream=None):
    """GDPA forward with fp8 (e4m3fn) Q and K standing for q8 * q_scale, k8 * k_scale; V and O bf16."""
    _check(load_library().gdpa_fp8_fwd(plan, _ptr(q8), _ptr(k8), _ptr(v), _ptr(q_off_dev), _ptr(kv_off_dev), B, H, d,
                                       _enum(act, ACT), window, float(q_scale), float(k_scale), _ptr(o),
                                       _stream(stream)))


def gdpa_fp8_bwd(plan, q8, k8, v, do8, q_off_dev, kv_off_dev, B, H, d, act, window, q_scale, k_scale, do_scale,
                 dq, dk, dv, stream=None):
    """GDPA backward with fp8 (e4m3fn) Q, K, dO standing for q8 * q_scale, k8 * k_scale, do8 * do_scale; V bf16."""
    _check(load_library().gdpa_fp8_bwd(plan, _ptr(q8), _ptr(k8), _ptr(v), _ptr(do8), _ptr(q_off_dev),
                                       _ptr(kv_off_dev), B, H, d, _enum(act, ACT), window, float(q_scale),
                                       float(k_scale), float(do_scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                       _stream(stream)))


def gdpa_norm_rstd(plan, q, k, v, H, d, norm, rstd, stream=None):
    """RMSNorm-prologue pre-pass: rstd (fp32, H (Tq + 2 Tk)) = 1/rms of the rows of the tensors in `norm`."""
    _check(load_library().gdpa_norm_rstd(plan, _ptr(q), _ptr(k), _ptr(v), H, d, norm_code(norm), _ptr(rstd),
                                         _stream(stream)))


def gdpa_norm_fwd(plan, q, k, v, q_off_dev, kv_off_dev, B, H, d, act, window, norm, rstd, o, stream=None):
    """GDPA on the RMS-normalised tensors in `norm`, from the raw tensors and gdpa_norm_rstd's factors."""
    _check(load_library().gdpa_norm_fwd(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(q_off_dev), _ptr(kv_off_dev), B, H,
                                        d, _enum(act, ACT), window, norm_code(norm), _ptr(rstd), _ptr(o),
                                        _stream(stream)))


def gdpa_norm_bwd(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, act, window, norm, rstd, dq, dk, dv,
                  stream=None):
    """Raw-input gradients of gdpa_norm_fwd."""
    _check(load_library().gdpa_norm_bwd(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(q_off_dev),
                                        _ptr(kv_off_dev), B, H, d, _enum(act, ACT), window, norm_code(norm),
                                        _ptr(rstd), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)))


def gdpa_norm_bwd_dkdv(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, act, window, norm, rstd, dk, dv,
                       stream=None):
    _check(load_library().gdpa_norm_bwd_dkdv(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(q_off_dev),
                                             _ptr(kv_off_dev), B, H, d, _enum(act, ACT), window, norm_code(norm),
                                             _ptr(rstd), _ptr(dk), _ptr(dv), _stream(stream)))


def gdpa_norm_bwd_dq(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, act, window, norm, rstd, dq, stream=None):
    _check(load_library().gdpa_norm_bwd_dq(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(q_off_dev),
                                           _ptr(kv_off_dev), B, H, d, _enum(act, ACT), window, norm_code(norm),
                                           _ptr(rstd), _ptr(dq), _stream(stream)))


CLAIM = {"auto": 0, "bins": 1, "always": 2}
SLOT_TIME = {"auto": 0, "off": 1}
DQ_TEAM = {"auto": 0, "one_wave": 1}


def _opts(host_only, bins, team, blocks, deal, split, unfused, store_ds=True, claim="auto", slot_time="auto",
          dq_team="auto"):
    return gdpa_plan_opts(int(host_only), (ctypes.c_int * 3)(*bins), (ctypes.c_int * 3)(*team),
                          (ctypes.c_int * 3)(*blocks), _enum(deal, DEAL), int(not split), int(unfused),
                          int(not store_ds), _enum(claim, CLAIM), _enum(slot_time, SLOT_TIME),
                          _enum(dq_team, DQ_TEAM))


def gdpa_pffn_plan_create(Tq: int, M: int, H: int, d: int, dtype, host_only: bool = False, bins=(0, 0, 0),
                          team=(0, 0, 0), blocks=(0, 0, 0), deal="greedy", split: bool = True,
                          unfused: bool = False, stream=None) -> int:
    """Plan of pFFN over Tq query rows and M shared weight rows (opaque handle)."""
    opts = _opts(host_only, bins, team, blocks, deal, split, unfused)
    out = _vp()
    _check(load_library().gdpa_pffn_plan_create(Tq, M, H, d, _enum(dtype, DTYPE), ctypes.byref(opts),
                                                None if host_only else _stream(stream), ctypes.byref(out)))
    return out.value


def gdpa_mx_fwd(plan, q8, q_scale, k8, k_scale, v, q_off_dev, kv_off_dev, B, H, d, act, window, o, stream=None):
    """Forward with block-scaled fp8 Q, K: e4m3 bytes [T, H, d] and E8M0 scale bytes [H, T, d / 32]."""
    _check(load_library().gdpa_mx_fwd(plan, _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v),
                                      _ptr(q_off_dev), _ptr(kv_off_dev), B, H, d, _enum(act, ACT), window, _ptr(o),
                                      _stream(stream)))


def gdpa_pffn_fwd(plan, q, wk, wv, act, o, stream=None):
    _check(load_library().gdpa_pffn_fwd(plan, _ptr(q), _ptr(wk), _ptr(wv), _enum(act, ACT), _ptr(o),
                                        _stream(stream)))


def gdpa_pffn_bwd(plan, q, wk, wv, dout, act, dq, dwk, dwv, stream=None):
    _check(load_library().gdpa_pffn_bwd(plan, _ptr(q), _ptr(wk), _ptr(wv), _ptr(dout), _enum(act, ACT),
                                        _ptr(dq), _ptr(dwk), _ptr(dwv), _stream(stream)))


def gdpa_plan_export(plan, list_) -> np.ndarray:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.gdpa_plan_export(plan, _enum(list_, LIST), None, ctypes.byref(n)))
    buf = np.zeros(n.value, dtype=np.int32)
    _check(lib.gdpa_plan_export(plan, _enum(list_, LIST), buf.ctypes.data, ctypes.byref(n)))
    return buf


def gdpa_plan_stats(plan) -> dict:
    st = gdpa_plan_stats_t()
    _check(load_library().gdpa_plan_stats(plan, ctypes.byref(st)))
    out = {}
    for name, _ in gdpa_plan_stats_t._fields_:
        val = getattr(st, name)
        out[name] = list(val) if hasattr(val, "__len__") else int(val)
    return out


def gdpa_plan_destroy(plan):
    if plan:
        load_library().gdpa_plan_destroy(plan)


def gdpa_status_string(status: int) -> str:
    return load_library().gdpa_status_string(status).decode()


def gdpa_last_error() -> str:
    return load_library().gdpa_last_error().decode()


def gdpa_gelu_poly_bound() -> float:
    return float(load_library().gdpa_gelu_poly_bound())


def gdpa_gelu_poly_grad_bound() -> float:
    return float(load_library().gdpa_gelu_poly_grad_bound())


# ---------------------------------------------------------------------------
# convenience: a plan object that allocates outputs with torch
# ---------------------------------------------------------------------------

class Plan:
    """Owns a plan; ``fwd`` / ``bwd`` allocate outputs (torch) and call the library."""

    def __init__(self, q_off_host, kv_off_host, H: int, d: int, window: int = 0, dtype="bf16", **opts):
        self.q_off = np.asarray(q_off_host, dtype=np.int32)
        self.kv_off = np.asarray(kv_off_host, dtype=np.int32)
        self.B = len(self.q_off) - 1
        self.H, self.d, self.window, self.dtype = H, d, window, dtype
        self.handle = gdpa_plan_create(self.q_off, self.kv_off, self.B, H, d, window, dtype, **opts)

    def close(self):
        if self.handle:
            gdpa_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def stats(self) -> dict:
        return gdpa_plan_stats(self.handle)

    def export(self, list_) -> np.ndarray:
        return gdpa_plan_export(self.handle, list_)

    def _out_dtype(self):
        import torch
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def _in_dtype(self):
        import torch
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def _check_tensor(self, name, t, rows, dtype, device=None):
        """Refuse, before any launch, a tensor the kernels would misread: not a
        contiguous [rows, H, d] tensor of `dtype` on a GPU (or on `device`)."""
        if t is None or not hasattr(t, "data_ptr"):
            raise TypeError(f"{name} must be a torch tensor")
        if tuple(t.shape) != (rows, self.H, self.d):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, the plan needs {(rows, self.H, self.d)}")
        if t.dtype != dtype:
            raise TypeError(f"{name} is {t.dtype}, the plan needs {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device.type != "cuda" or (device is not None and t.device != device):
            raise ValueError(f"{name} is on {t.device}, not on the inputs' GPU")

    def _check_offsets(self, q_off_dev, kv_off_dev, device):
        import torch
        for name, t in (("q_off_dev", q_off_dev), ("kv_off_dev", kv_off_dev)):
            if hasattr(t, "data_ptr"):
                if t.dtype != torch.int32 or tuple(t.shape) != (self.B + 1,) or not t.is_contiguous() \
                        or t.device != device:
                    raise ValueError(f"{name} must be a contiguous int32 [B + 1] tensor on {device}")

    def fwd(self, q, k, v, q_off_dev, kv_off_dev, act, o=None, stream=None):
        import torch
        Tq, Tk = int(self.q_off[-1]), int(self.kv_off[-1])
        self._check_tensor("q", q, Tq, self._in_dtype())
        dev = q.device
        self._check_tensor("k", k, Tk, self._in_dtype(), dev)
        self._check_tensor("v", v, Tk, self._in_dtype(), dev)
        self._check_offsets(q_off_dev, kv_off_dev, dev)
        if o is None:
            o = torch.empty(q.shape, dtype=self._out_dtype(), device=dev)
        self._check_tensor("o", o, Tq, self._out_dtype(), dev)
        gdpa_fwd(self.handle, q, k, v, q_off_dev, kv_off_dev, self.B, self.H, self.d, act, self.window, o,
                 stream)
        return o

    def bwd(self, q, k, v, dout, q_off_dev, kv_off_dev, act, dq=None, dk=None, dv=None, stream=None):
        import torch
        Tq, Tk = int(self.q_off[-1]), int(self.kv_off[-1])
        dt, it = self._out_dtype(), self._in_dtype()
        self._check_tensor("q", q, Tq, it)
        dev = q.device
        self._check_tensor("k", k, Tk, it, dev)
        self._check_tensor("v", v, Tk, it, dev)
        self._check_tensor("dout", dout, Tq, it, dev)
        self._check_offsets(q_off_dev, kv_off_dev, dev)
        dq = torch.empty(q.shape, dtype=dt, device=dev) if dq is None else dq
        dk = torch.empty(k.shape, dtype=dt, device=dev) if dk is None else dk
        dv = torch.empty(v.shape, dtype=dt, device=dev) if dv is None else dv
        self._check_tensor("dq", dq, Tq, dt, dev)
        self._check_tensor("dk", dk, Tk, dt, dev)
        self._check_tensor("dv", dv, Tk, dt, dev)
        gdpa_bwd(self.handle, q, k, v, dout, q_off_dev, kv_off_dev, self.B, self.H, self.d, act,
                 self.window, dq, dk, dv, stream)
        return dq, dk, dv
