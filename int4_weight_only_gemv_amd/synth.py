"""Seeded synthetic inputs for the int4 weight-only decode step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantization, no normalisation, no attention).  Both the
HIP path and the CPU oracle take their inputs from here, so the two sides see
identical data while sharing no code.

Workloads (model shapes after the kaminari page, "kaminari - a single-GPU Qwen3-VL
inference engine, explained", sections 01 and 04; dims of the Qwen3-VL-2B text
decoder):

  tiny      one tiny decoder layer, batch 1 (hidden 256, 4/2 heads, head_dim 64)
  layer     one full-size decoder layer, batch 1, 600 cached positions
  step      28-layer decoder + bf16 lm_head, batch 1, cache_position 700
  batch4    same model, 4 continuous-batching rows, one finished, 64 steps
  long16    same model, 16 rows, 8192-slot cache, 2048..8000 cached positions
  kv8       a reduced 2-layer decoder with the full model's head layout (16 q / 8
            kv heads, GQA 2) at head_dim 64, for parity runs of the kernels that
            give each XCD its own kv head

Two generators exist:
  * ``where="host"``: numpy PCG64 streams keyed by SeedSequence(base, spawn_key),
    so every tensor's draw is independent of the order tensors are made in;
  * ``where="device"``: torch's device generator seeded from the same key, used
    for the multi-GB weights and caches of the full-size workloads.  Values then
    differ from the host draw, which is fine: a test or bench run draws once and
    hands copies of the same tensors to both sides.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Dims:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    n_layers: int
    group_size: int
    mrope_section: Tuple[int, int, int]
    rms_eps: float = 1e-6
    rope_theta: float = 5_000_000.0
    mrope_interleaved: int = 1
    pad_id: int = 0
    eos_id: int = -1

    @property
    def qkv_rows(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim


TINY = Dims(hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=768,
            vocab=1024, n_layers=1, group_size=64, mrope_section=(12, 10, 10))
KV8 = Dims(hidden=512, n_heads=16, n_kv_heads=8, head_dim=64, intermediate=2048,
           vocab=2048, n_layers=2, group_size=64, mrope_section=(12, 10, 10))
QWEN3VL_2B = Dims(hidden=2048, n_heads=16, n_kv_heads=8, head_dim=128,
                  intermediate=6144, vocab=151936, n_layers=28, group_size=128,
                  mrope_section=(24, 20, 20))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # workload number; the base seed derives from it
    dims: Dims
    batch: int
    max_len: int
    steps: int
    description: str


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 0, TINY, 1, 128, 1,
                     "tiny single layer, batch 1, 16 cached positions"),
    "layer": Workload("layer", 1, dataclasses.replace(QWEN3VL_2B, n_layers=1, vocab=0),
                      1, 1024, 1, "one Qwen3-VL-2B-shaped layer, batch 1, 600 cached positions"),
    "step": Workload("step", 2, QWEN3VL_2B, 1, 1024, 1,
                     "28-layer Qwen3-VL-2B-shaped decoder + lm_head, batch 1, cache_position 700"),
    "batch4": Workload("batch4", 3, QWEN3VL_2B, 4, 1024, 64,
                       "28 layers, 4 slots (row 3 finished), 64 greedy steps"),
    "long16": Workload("long16", 4, QWEN3VL_2B, 16, 8192, 32,
                       "28 layers, 16 slots, 8192-slot cache, 2048..8000 cached positions"),
    "kv8": Workload("kv8", 5, KV8, 4, 384, 4,
                    "reduced 2-layer decoder with 8 kv heads, 4 slots, 384-slot cache"),
}


def base_seed(w: Workload) -> int:
    return 1000 * (w.index + 1) + 1


# tensor ids for spawn keys
T_IN_NORM, T_Q_NORM, T_K_NORM, T_POST_NORM, T_WQKV, T_WO, T_WGU, T_WD = range(8)
T_EMBED, T_FINAL_NORM, T_LM_HEAD, T_KCACHE, T_VCACHE, T_IDS, T_POS, T_CPOS, T_HIDDEN = range(8, 17)
GLOBAL_LAYER = 10_000


def _seed_seq(seed: int, layer: int, tensor: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(seed, spawn_key=(layer, tensor))


def _np_rng(seed: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_seed_seq(seed, layer, tensor)))


def _torch_seed(seed: int, layer: int, tensor: int) -> int:
    return int(_seed_seq(seed, layer, tensor).generate_state(1, np.uint64)[0] % (2**63 - 1))


def normal_bf16(shape, std: float, seed: int, layer: int, tensor: int,
                where: str = "host", device: Optional[str] = None) -> torch.Tensor:
    """N(0, std) draws rounded (RNE, by torch's cast) to bfloat16."""
    if where == "host":
        a = _np_rng(seed, layer, tensor).standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        return torch.from_numpy(a).to(torch.bfloat16)
    g = torch.Generator(device=device).manual_seed(_torch_seed(seed, layer, tensor))
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=g)
    return t.to(torch.bfloat16)


def uniform_bf16(shape, lo: float, hi: float, seed: int, layer: int, tensor: int) -> torch.Tensor:
    a = _np_rng(seed, layer, tensor).uniform(lo, hi, size=shape).astype(np.float32)
    return torch.from_numpy(a).to(torch.bfloat16)


def layer_weights(dims: Dims, seed: int, layer: int, where: str = "host",
                  device: Optional[str] = None) -> Dict[str, torch.Tensor]:
    """bf16 source weights of one decoder layer (before int4 quantization).

    Fused QKV rows are [q heads ; k heads ; v heads]; fused gate-up rows are
    [gate ; up].  Norm gains are U[0.5, 1.5] so a dropped gain is visible.
    """
    H, D, I = dims.hidden, dims.head_dim, dims.intermediate
    out = {
        "in_norm": uniform_bf16((H,), 0.5, 1.5, seed, layer, T_IN_NORM),
        "q_norm": uniform_bf16((D,), 0.5, 1.5, seed, layer, T_Q_NORM),
        "k_norm": uniform_bf16((D,), 0.5, 1.5, seed, layer, T_K_NORM),
        "post_norm": uniform_bf16((H,), 0.5, 1.5, seed, layer, T_POST_NORM),
        "wqkv": normal_bf16((dims.qkv_rows, H), 0.02, seed, layer, T_WQKV, where, device),
        "wo": normal_bf16((H, dims.n_heads * D), 0.02, seed, layer, T_WO, where, device),
        "wgu": normal_bf16((2 * I, H), 0.02, seed, layer, T_WGU, where, device),
        "wd": normal_bf16((H, I), 0.02, seed, layer, T_WD, where, device),
    }
    if where != "host":
        for k in ("in_norm", "q_norm", "k_norm", "post_norm"):
            out[k] = out[k].to(device)
    return out


def model_globals(dims: Dims, seed: int, where: str = "host",
                  device: Optional[str] = None) -> Dict[str, torch.Tensor]:
    """Untied bf16 embedding and lm_head, N(0, 0.02); final norm gain U[0.5, 1.5]."""
    V, H = dims.vocab, dims.hidden
    out = {
        "embed": normal_bf16((V, H), 0.02, seed, GLOBAL_LAYER, T_EMBED, where, device),
        "final_norm": uniform_bf16((H,), 0.5, 1.5, seed, GLOBAL_LAYER, T_FINAL_NORM),
        "lm_head": normal_bf16((V, H), 0.02, seed, GLOBAL_LAYER, T_LM_HEAD, where, device),
    }
    if where != "host":
        out["final_norm"] = out["final_norm"].to(device)
    return out


def kv_cache(dims: Dims, seed: int, batch: int, max_len: int, where: str = "host",
             device: Optional[str] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Static K and V caches, bf16 [L][B][Hkv][M][D], every slot N(0, 1).

    Slots at or beyond a row's cache_position hold seeded noise too: a correct
    step never reads them before writing, so any leak shows up in parity, and a
    stray write shows up in a byte compare.
    """
    shape = (dims.n_layers, batch, dims.n_kv_heads, max_len, dims.head_dim)
    k = normal_bf16(shape, 1.0, seed, GLOBAL_LAYER, T_KCACHE, where, device)
    v = normal_bf16(shape, 1.0, seed, GLOBAL_LAYER, T_VCACHE, where, device)
    return k, v


def step_inputs(w: Workload) -> Dict[str, np.ndarray]:
    """Token ids [B], 3-axis positions [3,B], cache positions [B], finished [B]."""
    seed, B, d = base_seed(w), w.batch, w.dims
    rng_ids = _np_rng(seed, GLOBAL_LAYER, T_IDS)
    rng_pos = _np_rng(seed, GLOBAL_LAYER, T_POS)
    rng_c = _np_rng(seed, GLOBAL_LAYER, T_CPOS)
    vocab = d.vocab if d.vocab > 0 else 1
    ids = rng_ids.integers(0, vocab, size=B, dtype=np.int64).astype(np.int32)
    finished = np.zeros(B, dtype=np.uint8)
    if w.name == "tiny":
        cpos = np.full(B, 16, np.int32)
        pos = rng_pos.integers(0, 64, size=(3, B)).astype(np.int32)
    elif w.name == "layer":
        cpos = np.full(B, 600, np.int32)
        pos = rng_pos.integers(0, 601, size=(3, B)).astype(np.int32)
    elif w.name == "step":
        # 512 visual tokens laid out as a 16x32 grid at slots [16, 528): text after the
        # image continues from max(t,h,w) + 1 of the image, so the token at slot 700
        # sits at 700 - 512 + 32 on all three axes.
        cpos = np.full(B, 700, np.int32)
        pos = np.full((3, B), 700 - 512 + 32, np.int32)
    elif w.name == "batch4":
        cpos = rng_c.integers(64, 1001, size=B).astype(np.int32)
        pos = np.stack([rng_pos.integers(0, int(c) + 1, size=3) for c in cpos], axis=1).astype(np.int32)
        finished[B - 1] = 1
        ids[B - 1] = d.pad_id
    elif w.name == "long16":
        cpos = rng_c.integers(2048, 8001, size=B).astype(np.int32)
        pos = np.stack([cpos, cpos, cpos]).astype(np.int32)
    elif w.name == "kv8":
        # split edges of 128-position attention splits, and the last slot
        cpos = np.array([0, 127, 128, 383], np.int32)[:B]
        pos = np.stack([rng_pos.integers(0, int(c) + 1, size=3) for c in cpos], axis=1).astype(np.int32)
    else:
        raise ValueError(w.name)
    return {"ids": ids, "positions": np.ascontiguousarray(pos), "cache_position": cpos,
            "finished": finished}


def hidden_input(dims: Dims, seed: int, batch: int) -> torch.Tensor:
    """Layer input for the single-layer workloads: N(0,1) rounded to bf16, held as fp32."""
    return normal_bf16((batch, dims.hidden), 1.0, seed, GLOBAL_LAYER, T_HIDDEN).float()
