"""CPU oracle for the int4 weight-only decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
binding) never does, and it shares no code with it.

The arithmetic lives in ``kmr_oracle.c`` (plain C, fp64, one dot product per
output); ``prefill.py`` holds a second, matrix-form implementation of the same
layer used only to pin the decode step (decode at position t equals the last row
of a full causal forward over tokens 0..t).  This module only marshals numpy
arrays into the C calls.

Parity notes: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, invariants or library routines; the
throughput figures it produces are a CPU baseline, not a parity claim.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional

import numpy as np

from . import build as _build

_LIB: Optional[C.CDLL] = None

_i64, _i32, _f64 = C.c_int64, C.c_int32, C.c_double
_p = C.c_void_p


class OraDims(C.Structure):
    _fields_ = [("hidden", _i64), ("n_heads", _i64), ("n_kv_heads", _i64), ("head_dim", _i64),
                ("intermediate", _i64), ("vocab", _i64), ("n_layers", _i64), ("group_size", _i64),
                ("rms_eps", _f64), ("rope_theta", _f64), ("mrope_section", _i32 * 3),
                ("mrope_interleaved", _i32), ("pad_id", _i32), ("eos_id", _i32)]


class OraQMat(C.Structure):
    _fields_ = [("packed", _p), ("sz", _p), ("N", _i64), ("K", _i64)]


class OraLayer(C.Structure):
    _fields_ = [("in_norm", _p), ("q_norm", _p), ("k_norm", _p), ("post_norm", _p),
                ("qkv", OraQMat), ("o", OraQMat), ("gate_up", OraQMat), ("down", OraQMat)]


class OraModel(C.Structure):
    _fields_ = [("embed", _p), ("final_norm", _p), ("lm_head", _p), ("layers", C.POINTER(OraLayer))]


ORA_ADVANCE = 1


def lib() -> C.CDLL:
    global _LIB
    if _LIB is None:
        path = _build.build(force=False)
        L = C.CDLL(path)
        L.ora_quantize_int4.argtypes = [_p, _i64, _i64, _i64, _p, _p]
        L.ora_dequant.argtypes = [_p, _p, _i64, _i64, _i64, _p]
        L.ora_gemv_int4.argtypes = [_p, _p, _i64, _i64, _i64, _p, _i64, _p]
        L.ora_rmsnorm.argtypes = [_p, _p, _i64, _f64, _p]
        L.ora_mrope_axis.argtypes = [_i64, _i64, _p, _i32]
        L.ora_mrope_axis.restype = _i32
        L.ora_mrope.argtypes = [_p, _i64, _p, _p, _i32, _f64]
        L.ora_attend.argtypes = [_p, _p, _p, _i64, _i64, _p]
        L.ora_bf16_round.argtypes = [_f64]
        L.ora_bf16_round.restype = _f64
        L.ora_silu.argtypes = [_f64]
        L.ora_silu.restype = _f64
        L.ora_decode_layer.argtypes = [C.POINTER(OraDims), C.POINTER(OraLayer), _i64, _p, _p,
                                       _i64, _i64, _p, _p, _p]
        L.ora_decode_step.argtypes = [C.POINTER(OraDims), C.POINTER(OraModel), _p, _p, _i64, _i64,
                                      _p, _p, _p, _p, C.c_uint32, _p, _p, _p, _p]
        L.ora_threads.restype = C.c_int
        _LIB = L
    return _LIB


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def as_u16(t) -> np.ndarray:
    """bf16 torch tensor (any device) -> host uint16 array of the same bits."""
    import torch
    if isinstance(t, np.ndarray):
        return _c(t, np.uint16)
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def threads() -> int:
    return int(lib().ora_threads())


def quantize_int4(w_u16: np.ndarray, group: int):
    w = _c(w_u16, np.uint16)
    N, K = w.shape
    packed = np.zeros((N, K // 2), np.uint8)
    sz = np.zeros((N, K // group, 2), np.uint16)
    lib().ora_quantize_int4(_ptr(w), N, K, group, _ptr(packed), _ptr(sz))
    return packed, sz


def dequant(packed: np.ndarray, sz: np.ndarray, group: int) -> np.ndarray:
    packed, sz = _c(packed, np.uint8), _c(sz, np.uint16)
    N, K = packed.shape[0], packed.shape[1] * 2
    out = np.empty((N, K), np.float64)
    lib().ora_dequant(_ptr(packed), _ptr(sz), N, K, group, _ptr(out))
    return out


def gemv_int4(packed: np.ndarray, sz: np.ndarray, group: int, x: np.ndarray) -> np.ndarray:
    packed, sz = _c(packed, np.uint8), _c(sz, np.uint16)
    x = _c(np.atleast_2d(x), np.float64)
    N, K = packed.shape[0], packed.shape[1] * 2
    y = np.empty((x.shape[0], N), np.float64)
    lib().ora_gemv_int4(_ptr(packed), _ptr(sz), N, K, group, _ptr(x), x.shape[0], _ptr(y))
    return y


def rmsnorm(x: np.ndarray, gain_u16: np.ndarray, eps: float) -> np.ndarray:
    x, g = _c(x, np.float64), _c(gain_u16, np.uint16)
    out = np.empty_like(x)
    lib().ora_rmsnorm(_ptr(x), _ptr(g), x.shape[-1], eps, _ptr(out))
    return out


def mrope_axis(j: int, half: int, sections, interleaved: int) -> int:
    s = _c(sections, np.int32)
    return int(lib().ora_mrope_axis(j, half, _ptr(s), interleaved))


def mrope(v: np.ndarray, pos3, sections, interleaved: int, theta: float) -> np.ndarray:
    out = _c(v, np.float64).copy()
    p, s = _c(pos3, np.int32), _c(sections, np.int32)
    lib().ora_mrope(_ptr(out), out.shape[-1], _ptr(p), _ptr(s), interleaved, theta)
    return out


def attend(q: np.ndarray, k_u16: np.ndarray, v_u16: np.ndarray) -> np.ndarray:
    q, k, v = _c(q, np.float64), _c(k_u16, np.uint16), _c(v_u16, np.uint16)
    out = np.empty(q.shape[-1], np.float64)
    lib().ora_attend(_ptr(q), _ptr(k), _ptr(v), k.shape[0], q.shape[-1], _ptr(out))
    return out


def bf16_round(x: float) -> float:
    return float(lib().ora_bf16_round(float(x)))


def silu(x: float) -> float:
    return float(lib().ora_silu(float(x)))


def make_dims(dims) -> OraDims:
    d = OraDims()
    for f in ("hidden", "n_heads", "n_kv_heads", "head_dim", "intermediate", "vocab",
              "n_layers", "group_size", "mrope_interleaved", "pad_id", "eos_id"):
        setattr(d, f, int(getattr(dims, f)))
    d.rms_eps = float(dims.rms_eps)
    d.rope_theta = float(dims.rope_theta)
    for i in range(3):
        d.mrope_section[i] = int(dims.mrope_section[i])
    return d


class Model:
    """Host copy of a quantized model for the oracle: the oracle quantizes the
    bf16 source weights itself (no input ever comes from the HIP path)."""

    def __init__(self, dims, layers: List[Dict], globals_: Optional[Dict] = None):
        self.dims = dims
        self.cdims = make_dims(dims)
        G = dims.group_size
        self._keep = []
        self.q = []
        self.clayers = (OraLayer * len(layers))()
        for i, w in enumerate(layers):
            ql = {}
            for name in ("in_norm", "q_norm", "k_norm", "post_norm"):
                ql[name] = as_u16(w[name])
            for name in ("wqkv", "wo", "wgu", "wd"):
                if name + "_packed" in w:
                    ql[name] = (_c(w[name + "_packed"], np.uint8), _c(w[name + "_sz"], np.uint16))
                else:
                    ql[name] = quantize_int4(as_u16(w[name]), G)
            self.q.append(ql)
            cl = self.clayers[i]
            cl.in_norm, cl.q_norm = _ptr(ql["in_norm"]), _ptr(ql["q_norm"])
            cl.k_norm, cl.post_norm = _ptr(ql["k_norm"]), _ptr(ql["post_norm"])
            for field, name in (("qkv", "wqkv"), ("o", "wo"), ("gate_up", "wgu"), ("down", "wd")):
                pk, sz = ql[name]
                m = getattr(cl, field)
                m.packed, m.sz, m.N, m.K = _ptr(pk), _ptr(sz), pk.shape[0], pk.shape[1] * 2
        self.g = None
        if globals_ is not None:
            self.g = {k: as_u16(v) for k, v in globals_.items()}
            self.cmodel = OraModel(_ptr(self.g["embed"]), _ptr(self.g["final_norm"]),
                                   _ptr(self.g["lm_head"]), self.clayers)

    def decode_layer(self, layer: int, kc: np.ndarray, vc: np.ndarray, x: np.ndarray,
                     pos: np.ndarray, cpos: np.ndarray, layer_index_in_cache: Optional[int] = None):
        """In place on x [B,H] (fp64), kc/vc uint16 [L][B][Hkv][M][D]."""
        B, M = kc.shape[1], kc.shape[3]
        li = layer if layer_index_in_cache is None else layer_index_in_cache
        assert x.dtype == np.float64 and x.flags.c_contiguous
        pos, cpos = _c(pos, np.int32), _c(cpos, np.int32)
        rc = lib().ora_decode_layer(C.byref(self.cdims), C.byref(self.clayers[layer]), li,
                                    _ptr(kc), _ptr(vc), B, M, _ptr(x), _ptr(pos), _ptr(cpos))
        if rc:
            raise ValueError(f"oracle decode_layer rejected the call (rc={rc})")
        return x

    def decode_step(self, kc: np.ndarray, vc: np.ndarray, ids, pos: np.ndarray, cpos: np.ndarray,
                    finished: Optional[np.ndarray] = None, advance: bool = False,
                    want_logits: bool = True):
        """One greedy step.  pos/cpos/finished are updated in place when advancing.
        Returns dict(next, logits, margin, hidden)."""
        assert self.g is not None
        d = self.dims
        B, M = kc.shape[1], kc.shape[3]
        ids = _c(ids, np.int32)
        assert pos.dtype == np.int32 and cpos.dtype == np.int32
        nxt = np.empty(B, np.int32)
        logits = np.empty((B, d.vocab), np.float64) if want_logits else None
        margin = np.empty(B, np.float64)
        hidden = np.empty((B, d.hidden), np.float64)
        rc = lib().ora_decode_step(C.byref(self.cdims), C.byref(self.cmodel), _ptr(kc), _ptr(vc),
                                   B, M, _ptr(ids), _ptr(pos), _ptr(cpos), _ptr(finished),
                                   ORA_ADVANCE if advance else 0, _ptr(nxt), _ptr(logits),
                                   _ptr(margin), _ptr(hidden))
        if rc:
            raise ValueError(f"oracle decode_step rejected the call (rc={rc})")
        return {"next": nxt, "logits": logits, "margin": margin, "hidden": hidden}
