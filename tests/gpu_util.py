"""Shared helpers for the GPU parity tests: build the same seeded model and cache
for the HIP path and for the oracle, and the error metrics.

Inputs always come from int4_weight_only_gemv_amd.synth; the oracle quantizes
the bf16 source weights itself, so no oracle input comes from the HIP path.
"""
from __future__ import annotations

import dataclasses
import sys
from typing import Dict, List

import numpy as np
import torch

import oracle
from int4_weight_only_gemv_amd import synth

TOL = 2e-2           # max relative error on hidden states, logits and written K/V
MARGIN = 1e-2        # tokens must agree where the oracle's top-2 margin exceeds this


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def max_rel(got, ref) -> float:
    """Largest absolute error over the largest reference magnitude, per row, worst row."""
    got = np.atleast_2d(np.asarray(got, np.float64))
    ref = np.atleast_2d(np.asarray(ref, np.float64))
    num = np.abs(got - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max())


def bf16_host(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_device_bf16(u16: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(device).view(torch.bfloat16)


@dataclasses.dataclass
class Pair:
    dims: synth.Dims
    dev: object            # kmr.DeviceModel
    ora: oracle.Model


def build_pair(dims: synth.Dims, seed: int, where: str, with_globals: bool) -> Pair:
    """Same seeded weights for both sides.  where="host": numpy draws (small models);
    where="device": torch device draws, copied to the host for the oracle."""
    from int4_weight_only_gemv_amd import kmr
    host_layers: List[Dict] = []
    dev_layers: List[Dict] = []
    for l in range(dims.n_layers):
        w = synth.layer_weights(dims, seed, l, where=where, device="cuda" if where == "device" else None)
        host_layers.append({k: oracle.as_u16(v) for k, v in w.items()})
        dev_layers.append(w)
    glob = None
    if with_globals:
        glob = synth.model_globals(dims, seed, where=where, device="cuda" if where == "device" else None)
    dev = kmr.DeviceModel(dims, dev_layers, glob)
    del dev_layers
    ora = oracle.Model(dims, host_layers, None if glob is None else {k: oracle.as_u16(v) for k, v in glob.items()})
    del host_layers
    torch.cuda.empty_cache()
    return Pair(dims, dev, ora)


def make_caches(dims: synth.Dims, seed: int, batch: int, max_len: int, where: str,
                host_rows=None):
    """Device KVCache plus host (uint16) copies of the rows the oracle will run."""
    from int4_weight_only_gemv_amd import kmr
    cfg = kmr.make_config(dims)
    kv = kmr.KVCache(cfg, batch, max_len, zero=False)
    k, v = synth.kv_cache(dims, seed, batch, max_len, where=where,
                          device="cuda" if where == "device" else None)
    kv.k.copy_(k)
    kv.v.copy_(v)
    del k, v
    rows = list(range(batch)) if host_rows is None else list(host_rows)
    kh = oracle.as_u16(kv.k[:, rows].contiguous())
    vh = oracle.as_u16(kv.v[:, rows].contiguous())
    torch.cuda.synchronize()
    return kv, kh, vh
