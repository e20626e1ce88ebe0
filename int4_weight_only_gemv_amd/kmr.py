"""ctypes binding of libkmr.so (C ABI in include/kmr.h).

Argument marshalling only: torch provides device memory and the stream, every
step of the decode path runs in the library's HIP kernels.  Importing this module
fails loudly when the library is not built or would load a second HIP runtime;
there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence

import torch  # loads the HIP runtime that libkmr.so must share

HERE = os.path.dirname(os.path.abspath(__file__))
# KMR_LIBRARY may point at another build of the same library (e.g. a diagnostic build).
LIB_PATH = os.environ.get("KMR_LIBRARY", os.path.join(HERE, "libkmr.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m int4_weight_only_gemv_amd.build`")
_lib = C.CDLL(LIB_PATH)


def _hip_runtimes() -> List[str]:
    with open("/proc/self/maps") as f:
        return sorted({line.split()[-1] for line in f if "libamdhip64" in line})


if len(_hip_runtimes()) > 1:
    raise ImportError(f"two HIP runtimes are mapped: {_hip_runtimes()}")

KMR_OK, KMR_EINVAL, KMR_ESHAPE, KMR_ENOMEM, KMR_EHIP = 0, -1, -2, -3, -4
KMR_STATUS_CACHE_POS, KMR_STATUS_TOKEN, KMR_STATUS_TIMEOUT, KMR_STATUS_TOPOLOGY, KMR_STATUS_RANGE = 1, 2, 4, 8, 16
KMR_MAX_BATCH = 64
KMR_PREFILL_CHUNK = 512
KMR_ADVANCE = 1
KMR_MULTI_KERNEL = 2
KMR_DEVICE_WIDE = 4
KMR_COOPERATIVE = 8
KMR_BATCH_INVARIANT = 16
KMR_DEVICE_SCOPE_STORES = 32
KMR_CLEAR_WORKSPACE = 64
KMR_STATIC_WORKSPACE_BYTES = 48 << 20
KMR_TEST_STALL = 256

_i32, _p = C.c_int32, C.c_void_p


class Config(C.Structure):
    _fields_ = [("hidden", _i32), ("n_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32),
                ("intermediate", _i32), ("vocab", _i32), ("n_layers", _i32), ("group_size", _i32),
                ("rms_eps", C.c_float), ("rope_theta", C.c_double), ("mrope_section", _i32 * 3),
                ("mrope_interleaved", _i32), ("pad_id", _i32), ("eos_id", _i32)]


class QWeight(C.Structure):
    _fields_ = [("packed", _p), ("sz", _p), ("N", _i32), ("K", _i32)]


class Layer(C.Structure):
    _fields_ = [("in_norm", _p), ("q_norm", _p), ("k_norm", _p), ("post_norm", _p),
                ("qkv", QWeight), ("o", QWeight), ("gate_up", QWeight), ("down", QWeight)]


class Model(C.Structure):
    _fields_ = [("embed", _p), ("final_norm", _p), ("lm_head", _p), ("layers", C.POINTER(Layer))]


class KV(C.Structure):
    _fields_ = [("k", _p), ("v", _p), ("n_layers", _i32), ("batch", _i32), ("n_kv_heads", _i32),
                ("max_len", _i32), ("head_dim", _i32), ("bytes", C.c_size_t)]


_lib.kmr_kv_alloc.argtypes = [C.POINTER(Config), _i32, _i32, _p, C.c_size_t, _i32, _p, C.POINTER(KV)]
_lib.kmr_quantize_int4.argtypes = [_p, _i32, _i32, _i32, _p, _p, _p]
_lib.kmr_workspace_bytes.argtypes = [C.POINTER(Config), _i32, _i32]
_lib.kmr_workspace_bytes.restype = C.c_size_t
_lib.kmr_prefill_workspace_bytes.argtypes = [C.POINTER(Config), _i32, _i32]
_lib.kmr_prefill_workspace_bytes.restype = C.c_size_t
_lib.kmr_workspace_init.argtypes = [_p, C.c_size_t, _p]
_lib.kmr_debug_stepx_fits.argtypes = [C.POINTER(Config), _i32, _i32]
_lib.kmr_decode_layer.argtypes = [C.POINTER(Config), C.POINTER(Layer), _i32, C.POINTER(KV), _p, _p,
                                  _p, _i32, _p, C.c_size_t, _p]
_lib.kmr_decode_step.argtypes = [C.POINTER(Config), C.POINTER(Model), C.POINTER(KV), _p, _p, _p, _p,
                                 _i32, _p, _p, C.c_uint32, _p, C.c_size_t, _p]
_lib.kmr_decode_step_static.argtypes = [C.POINTER(Config), C.POINTER(Model), C.POINTER(KV), _p, _p, _p, _p,
                                        _i32, _p, _p, C.c_uint32, _p]
_lib.kmr_decode_step_prefix.argtypes = [C.POINTER(Config), C.POINTER(Model), C.POINTER(KV), _p, _p, _p, _p,
                                        _i32, _p, _p, C.c_uint32, _i32, _p, C.c_size_t, _p]
_lib.kmr_prefill.argtypes = [C.POINTER(Config), C.POINTER(Model), C.POINTER(KV), _i32, _p, _p, _i32, _i32,
                             _p, _p, _p, C.c_size_t, _p]
_lib.kmr_status.argtypes = [_p, _p, C.POINTER(C.c_uint32)]
_lib.kmr_read_probe.argtypes = [_p, C.c_size_t, _p, _p]
_lib.kmr_kv_copy_row.argtypes = [C.POINTER(KV), _i32, C.POINTER(KV), _i32, _i32, _p]
_lib.kmr_slot_admit.argtypes = [_p, _p, _p, _p, _i32, _i32, _i32, C.POINTER(_i32), _i32, _p]
_lib.kmr_slot_retire.argtypes = [_p, _i32, _i32, _p]
_lib.kmr_strerror.restype = C.c_char_p
_lib.kmr_last_error.restype = C.c_char_p

EXPORTED = ["kmr_kv_alloc", "kmr_kv_copy_row", "kmr_quantize_int4", "kmr_workspace_bytes",
            "kmr_prefill_workspace_bytes", "kmr_debug_stepx_fits",
            "kmr_workspace_init", "kmr_decode_layer", "kmr_decode_step", "kmr_decode_step_static",
            "kmr_decode_step_prefix",
            "kmr_prefill",
            "kmr_slot_admit", "kmr_slot_retire", "kmr_status", "kmr_read_probe", "kmr_strerror",
            "kmr_last_error"]
KMR_READ_PROBE_THREADS = 256 * 8 * 256


def read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """kmr_read_probe: stream every byte of buf (device, contiguous) with 16-byte
    non-temporal loads; sink: uint32/int32 device tensor of KMR_READ_PROBE_THREADS."""
    assert sink.numel() >= KMR_READ_PROBE_THREADS and sink.element_size() == 4
    _check(_lib.kmr_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


class KmrError(RuntimeError):
    def __init__(self, code: int):
        self.code = code
        super().__init__(f"{_lib.kmr_strerror(code).decode()} ({code}): {_lib.kmr_last_error().decode()}")


def _check(rc: int) -> None:
    if rc != KMR_OK:
        raise KmrError(rc)


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("kmr takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("kmr takes contiguous tensors only")
    return t.data_ptr()


def make_config(dims) -> Config:
    c = Config()
    for f in ("hidden", "n_heads", "n_kv_heads", "head_dim", "intermediate", "vocab", "n_layers",
              "group_size", "mrope_interleaved", "pad_id", "eos_id"):
        setattr(c, f, int(getattr(dims, f)))
    c.rms_eps = float(dims.rms_eps)
    c.rope_theta = float(dims.rope_theta)
    for i in range(3):
        c.mrope_section[i] = int(dims.mrope_section[i])
    return c


def quantize_int4(w: torch.Tensor, group: int, stream=None):
    """bf16 [N,K] device tensor -> (packed uint8 [N,K/2], sz int16 [N,K/group,2] bf16 bits)."""
    if w.dtype != torch.bfloat16 or w.dim() != 2:
        raise ValueError("quantize_int4 takes a 2-D bfloat16 tensor")
    N, K = w.shape
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    sz = torch.empty((N, max(K // group, 1), 2), dtype=torch.int16, device=w.device)
    _check(_lib.kmr_quantize_int4(_ptr(w), N, K, group, _ptr(packed), _ptr(sz), _stream(stream)))
    return packed, sz


def workspace_bytes(cfg: Config, batch: int, max_len: int) -> int:
    return int(_lib.kmr_workspace_bytes(C.byref(cfg), batch, max_len))


def prefill_workspace_bytes(cfg: Config, n_tokens: int, max_len: int) -> int:
    return int(_lib.kmr_prefill_workspace_bytes(C.byref(cfg), n_tokens, max_len))


def debug_stepx_fits(cfg: Config, batch: int, n_groups: int) -> int:
    """kmr_debug_stepx_fits: 1 if the XCD-local persistent kernel takes this shape."""
    return int(_lib.kmr_debug_stepx_fits(C.byref(cfg), batch, n_groups))


class Workspace:
    def __init__(self, cfg: Config, batch: int, max_len: int, device="cuda", stream=None, nbytes=None):
        n = workspace_bytes(cfg, batch, max_len) if nbytes is None else nbytes
        if n == 0:
            raise KmrError(KMR_EINVAL)
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        _check(_lib.kmr_workspace_init(_ptr(self.buf), n, _stream(stream)))

    @classmethod
    def for_prefill(cls, cfg: Config, n_tokens: int, max_len: int, device="cuda", stream=None):
        """The workspace of a kmr_prefill of n_tokens (kmr_prefill_workspace_bytes)."""
        return cls(cfg, 0, max_len, device, stream,
                   nbytes=prefill_workspace_bytes(cfg, n_tokens, max_len))

    @property
    def ptr(self):
        return self.buf.data_ptr()

    @property
    def nbytes(self):
        return self.buf.numel()

    def init(self, stream=None) -> None:
        """kmr_workspace_init again (after an error or KMR_STATUS_TIMEOUT)."""
        _check(_lib.kmr_workspace_init(self.ptr, self.nbytes, _stream(stream)))

    def status(self, stream=None) -> int:
        v = C.c_uint32(0)
        _check(_lib.kmr_status(self.ptr, _stream(stream), C.byref(v)))
        return int(v.value)


class KVCache:
    """Static bf16 K/V [L][B][Hkv][M][D] bound to one torch allocation."""

    def __init__(self, cfg: Config, batch: int, max_len: int, device="cuda", zero=True, stream=None):
        self.desc = KV()
        _check(_lib.kmr_kv_alloc(C.byref(cfg), batch, max_len, None, 0, 0, None, C.byref(self.desc)))
        self.buf = torch.empty(self.desc.bytes, dtype=torch.uint8, device=device)
        _check(_lib.kmr_kv_alloc(C.byref(cfg), batch, max_len, _ptr(self.buf), self.buf.numel(),
                                 1 if zero else 0, _stream(stream), C.byref(self.desc)))
        shape = (cfg.n_layers, batch, cfg.n_kv_heads, max_len, cfg.head_dim)
        n = cfg.n_layers * batch * cfg.n_kv_heads * max_len * cfg.head_dim
        half = self.desc.bytes // 2
        self.k = self.buf[:half].view(torch.bfloat16)[:n].view(shape)
        self.v = self.buf[half:].view(torch.bfloat16)[:n].view(shape)


def kv_copy_row(dst: "KVCache", dst_row: int, src: "KVCache", src_row: int, n_positions: int,
                stream=None) -> None:
    """Positions [0, n_positions) of cache row src_row of src -> row dst_row of dst
    (every layer and kv head, K and V)."""
    _check(_lib.kmr_kv_copy_row(C.byref(dst.desc), dst_row, C.byref(src.desc), src_row, n_positions,
                                _stream(stream)))


def slot_admit(token_ids: torch.Tensor, positions: torch.Tensor, cache_position: torch.Tensor,
               finished: torch.Tensor, row: int, token: int, pos, cache_pos: int, stream=None) -> None:
    """Row `row` becomes live: its token id, three positions (t, h, w), cache position,
    and a cleared finished flag, set on the device."""
    p3 = (_i32 * 3)(*[int(v) for v in pos])
    _check(_lib.kmr_slot_admit(_ptr(token_ids), _ptr(positions), _ptr(cache_position), _ptr(finished),
                               int(token_ids.numel()), row, token, p3, cache_pos, _stream(stream)))


def slot_retire(finished: torch.Tensor, row: int, stream=None) -> None:
    """Row `row` is finished from the next step on."""
    _check(_lib.kmr_slot_retire(_ptr(finished), int(finished.numel()), row, _stream(stream)))


def _qweight(packed: torch.Tensor, sz: torch.Tensor) -> QWeight:
    return QWeight(_ptr(packed), _ptr(sz), packed.shape[0], packed.shape[1] * 2)


class DeviceModel:
    """Device-resident int4 decoder.  Quantization runs through kmr_quantize_int4
    on the bf16 source weights given (dicts as made by synth.layer_weights)."""

    def __init__(self, dims, layers: Sequence[Dict[str, torch.Tensor]],
                 globals_: Optional[Dict[str, torch.Tensor]] = None, device="cuda",
                 keep_source=False):
        self.dims = dims
        self.cfg = make_config(dims)
        G = dims.group_size
        self.tensors: List[Dict[str, torch.Tensor]] = []
        self.clayers = (Layer * len(layers))()
        for i, w in enumerate(layers):
            t = {k: w[k].to(device).contiguous() for k in ("in_norm", "q_norm", "k_norm", "post_norm")}
            for name in ("wqkv", "wo", "wgu", "wd"):
                src = w[name].to(device).contiguous()
                t[name + "_packed"], t[name + "_sz"] = quantize_int4(src, G)
                if keep_source:
                    t[name] = src
                del src
            self.tensors.append(t)
            cl = self.clayers[i]
            cl.in_norm, cl.q_norm = _ptr(t["in_norm"]), _ptr(t["q_norm"])
            cl.k_norm, cl.post_norm = _ptr(t["k_norm"]), _ptr(t["post_norm"])
            cl.qkv = _qweight(t["wqkv_packed"], t["wqkv_sz"])
            cl.o = _qweight(t["wo_packed"], t["wo_sz"])
            cl.gate_up = _qweight(t["wgu_packed"], t["wgu_sz"])
            cl.down = _qweight(t["wd_packed"], t["wd_sz"])
        self.globals = None
        if globals_ is not None:
            self.globals = {k: v.to(device).contiguous() for k, v in globals_.items()}
            self.cmodel = Model(_ptr(self.globals["embed"]), _ptr(self.globals["final_norm"]),
                                _ptr(self.globals["lm_head"]), self.clayers)

    def decode_layer(self, layer: int, kv: KVCache, hidden: torch.Tensor, positions: torch.Tensor,
                     cache_position: torch.Tensor, ws: Workspace, cache_layer: Optional[int] = None,
                     stream=None) -> torch.Tensor:
        """In place on hidden (fp32 [B,H] device).  positions int32 [3,B], cache_position int32 [B]."""
        assert hidden.dtype == torch.float32 and positions.dtype == torch.int32
        assert cache_position.dtype == torch.int32
        B = hidden.shape[0]
        li = layer if cache_layer is None else cache_layer
        _check(_lib.kmr_decode_layer(C.byref(self.cfg), C.byref(self.clayers[layer]), li,
                                     C.byref(kv.desc), _ptr(hidden), _ptr(positions),
                                     _ptr(cache_position), B, ws.ptr, ws.nbytes, _stream(stream)))
        return hidden

    def decode_step(self, kv: KVCache, token_ids: torch.Tensor, positions: torch.Tensor,
                    cache_position: torch.Tensor, next_ids: torch.Tensor, ws: Workspace,
                    finished: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                    advance: bool = False, multi_kernel: bool = False, device_wide: bool = False,
                    cooperative: bool = False, shared_prefix: int = 0, device_scope_stores: bool = False,
                    batch_invariant: bool = False, extra_flags: int = 0, stream=None) -> torch.Tensor:
        """shared_prefix > 0: kmr_decode_step_prefix (every row holds the same K/V in
        cache positions [0, shared_prefix); the per-phase kernels read it once).
        extra_flags: further KMR_* flag bits, passed through."""
        B = token_ids.shape[0]
        assert token_ids.dtype == torch.int32 and next_ids.dtype == torch.int32
        assert finished is None or finished.dtype == torch.uint8
        flags = ((KMR_ADVANCE if advance else 0) | (KMR_MULTI_KERNEL if multi_kernel else 0)
                 | (KMR_DEVICE_WIDE if device_wide else 0) | (KMR_COOPERATIVE if cooperative else 0)
                 | (KMR_DEVICE_SCOPE_STORES if device_scope_stores else 0)
                 | (KMR_BATCH_INVARIANT if batch_invariant else 0) | int(extra_flags))
        args = (C.byref(self.cfg), C.byref(self.cmodel), C.byref(kv.desc), _ptr(token_ids), _ptr(positions),
                _ptr(cache_position), _ptr(finished), B, _ptr(next_ids), _ptr(logits), flags)
        if shared_prefix:
            _check(_lib.kmr_decode_step_prefix(*args, shared_prefix, ws.ptr, ws.nbytes, _stream(stream)))
        else:
            _check(_lib.kmr_decode_step(*args, ws.ptr, ws.nbytes, _stream(stream)))
        return next_ids

    def decode_step_static(self, kv: KVCache, token_ids: torch.Tensor, positions: torch.Tensor,
                           cache_position: torch.Tensor, next_ids: torch.Tensor,
                           finished: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                           advance: bool = False, flags: int = 0, stream=None) -> torch.Tensor:
        """kmr_decode_step_static: the step with the library's static workspace (no
        workspace argument, nothing allocated).  flags: further KMR_* bits."""
        B = token_ids.shape[0]
        assert token_ids.dtype == torch.int32 and next_ids.dtype == torch.int32
        f = (KMR_ADVANCE if advance else 0) | int(flags)
        _check(_lib.kmr_decode_step_static(C.byref(self.cfg), C.byref(self.cmodel), C.byref(kv.desc),
                                           _ptr(token_ids), _ptr(positions), _ptr(cache_position), _ptr(finished),
                                           B, _ptr(next_ids), _ptr(logits), f, _stream(stream)))
        return next_ids

    def prefill(self, kv: KVCache, row: int, token_ids: torch.Tensor, positions: torch.Tensor, start: int,
                next_id: torch.Tensor, ws: Workspace, logits: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
        """kmr_prefill: token_ids [T] int32, positions [3, T] int32 (contiguous), the
        tokens at cache positions start..start+T-1 of cache row `row`; ws sized for
        Workspace.for_prefill(cfg, T, max_len)."""
        T = token_ids.shape[0]
        assert token_ids.dtype == torch.int32 and positions.dtype == torch.int32 and next_id.dtype == torch.int32
        assert positions.shape == (3, T) and positions.is_contiguous() and token_ids.is_contiguous()
        _check(_lib.kmr_prefill(C.byref(self.cfg), C.byref(self.cmodel), C.byref(kv.desc), row, _ptr(token_ids),
                                _ptr(positions), start, T, _ptr(next_id), _ptr(logits), ws.ptr, ws.nbytes,
                                _stream(stream)))
        return next_id
