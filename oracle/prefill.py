"""Full causal forward of the decoder over T tokens -- TEST INFRASTRUCTURE ONLY.

A second, matrix-form implementation of the same decoder layer as
``kmr_oracle.c`` (numpy, fp64, written separately: its own nibble unpacking, its
own RoPE as a complex rotation, its own GQA head repeat, a causal mask instead of
a cache window).  It exists to pin the one-token decode step: decoding token t
against a cache holding the K/V of tokens 0..t-1 must give the last row of this
forward over tokens 0..t (kaminari page, section 04: prefill writes the static
cache, then each decode step extends it by one token).

As in decode, K and V are rounded to bf16 (their storage precision) before
attention reads them.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np


def bf16_values(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even (normal range)."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    return (round_bf16(x).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def unpack_int4(packed: np.ndarray, sz: np.ndarray, group: int) -> np.ndarray:
    """Dense fp64 weights from codes (even k in the low nibble) and (scale, zero)."""
    packed = np.asarray(packed, np.uint8)
    N, K = packed.shape[0], packed.shape[1] * 2
    codes = np.empty((N, K), np.int64)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    s = bf16_values(sz[..., 0])            # [N, K/G]
    z = bf16_values(sz[..., 1])
    s_full = np.repeat(s, group, axis=1)
    z_full = np.repeat(z, group, axis=1)
    return (codes - 8) * s_full + z_full


def _rms(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * gain


def _axis_table(half: int, sections: Sequence[int], interleaved: int) -> np.ndarray:
    j = np.arange(half)
    if interleaved:
        ax = np.zeros(half, np.int64)
        ax[(j % 3 == 1) & (j < 3 * sections[1])] = 1
        ax[(j % 3 == 2) & (j < 3 * sections[2])] = 2
        return ax
    return np.where(j < sections[0], 0, np.where(j < sections[0] + sections[1], 1, 2))


def _rope(x: np.ndarray, pos3: np.ndarray, dims) -> np.ndarray:
    """x [T, heads, D]; pos3 [3, T]. Rotation of (x_j, x_{j+D/2}) as a complex number."""
    D = x.shape[-1]
    half = D // 2
    ax = _axis_table(half, dims.mrope_section, dims.mrope_interleaved)
    inv_freq = float(dims.rope_theta) ** (-2.0 * np.arange(half) / D)
    ang = pos3[ax, :].T.astype(np.float64) * inv_freq          # [T, half]
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * ang)[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1)


def forward(dims, layers: List[Dict[str, np.ndarray]], x0: np.ndarray, pos3: np.ndarray,
            ) -> Tuple[np.ndarray, List[Tuple[np.ndarray, np.ndarray]]]:
    """Causal forward of all layers over T tokens of ONE sequence.

    layers[i] holds uint16 gains ``in_norm, q_norm, k_norm, post_norm`` and int4
    matrices ``wqkv, wo, wgu, wd`` as (packed, sz) pairs.  x0 [T, H] fp64 is the
    embedded input; pos3 [3, T].  Returns the final hidden [T, H] (before the
    final norm) and per layer the bf16-rounded (K, V) [T, Hkv, D] as fp64.
    """
    Hq, Hkv, D, I, G = dims.n_heads, dims.n_kv_heads, dims.head_dim, dims.intermediate, dims.group_size
    eps = dims.rms_eps
    x = np.array(x0, np.float64)
    T = x.shape[0]
    kv = []
    causal = np.tril(np.ones((T, T), bool))
    for w in layers:
        wqkv = unpack_int4(*w["wqkv"], G)
        wo = unpack_int4(*w["wo"], G)
        wgu = unpack_int4(*w["wgu"], G)
        wd = unpack_int4(*w["wd"], G)
        h = _rms(x, bf16_values(w["in_norm"]), eps)
        qkv = h @ wqkv.T
        q = qkv[:, : Hq * D].reshape(T, Hq, D)
        k = qkv[:, Hq * D: (Hq + Hkv) * D].reshape(T, Hkv, D)
        v = qkv[:, (Hq + Hkv) * D:].reshape(T, Hkv, D)
        q = _rope(_rms(q, bf16_values(w["q_norm"]), eps), pos3, dims)
        k = _rope(_rms(k, bf16_values(w["k_norm"]), eps), pos3, dims)
        kb, vb = round_bf16(k), round_bf16(v)
        kv.append((kb, vb))
        rep = Hq // Hkv
        kr = np.repeat(kb, rep, axis=1)                  # [T, Hq, D]
        vr = np.repeat(vb, rep, axis=1)
        scores = np.einsum("thd,shd->hts", q, kr) / np.sqrt(D)   # [Hq, T, T]
        scores = np.where(causal[None], scores, -np.inf)
        scores -= scores.max(axis=-1, keepdims=True)
        p = np.exp(scores)
        p /= p.sum(axis=-1, keepdims=True)
        o = np.einsum("hts,shd->thd", p, vr).reshape(T, Hq * D)
        x = x + o @ wo.T
        h = _rms(x, bf16_values(w["post_norm"]), eps)
        gu = h @ wgu.T
        g, u = gu[:, :I], gu[:, I:]
        x = x + ((g / (1.0 + np.exp(-g))) * u) @ wd.T
    return x, kv


def logits(dims, x: np.ndarray, final_norm_u16: np.ndarray, lm_head_u16: np.ndarray) -> np.ndarray:
    h = _rms(x, bf16_values(final_norm_u16), dims.rms_eps)
    return h @ bf16_values(lm_head_u16).T
