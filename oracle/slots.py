"""Slot operations of a continuous-batching scheduler, as plain array updates --
TEST INFRASTRUCTURE ONLY (only tests/ may import it; the HIP library never does).

kaminari page, section 08 ("three schedulers, one engine"): the
ContinuousBatchScheduler admits requests into free DecodeSlots, each pinned to a
physical row of one shared static cache, ticks the active slots one token at a
time and finalizes a row the moment it finishes; copy_row_from moves a row's KV
state into another row.  Section 03 ("State model") lists what a live row carries:
the next-token column, the 3D positions, the cache position and the finished flag.

The caches are numpy arrays [n_layers][batch][n_kv_heads][max_len][head_dim] of
bf16 bit patterns (uint16), as the decode oracle takes them.
"""
from __future__ import annotations

import numpy as np


def kv_copy_row(dst_k: np.ndarray, dst_v: np.ndarray, dst_row: int, src_k: np.ndarray,
                src_v: np.ndarray, src_row: int, n_positions: int) -> None:
    """Positions [0, n_positions) of row src_row -> row dst_row, every layer and kv head."""
    n = int(n_positions)
    if not (0 <= n <= min(dst_k.shape[3], src_k.shape[3])):
        raise ValueError("n_positions outside both caches")
    dst_k[:, dst_row, :, :n, :] = src_k[:, src_row, :, :n, :]
    dst_v[:, dst_row, :, :n, :] = src_v[:, src_row, :, :n, :]


def slot_admit(token_ids: np.ndarray, positions: np.ndarray, cache_position: np.ndarray,
               finished: np.ndarray, row: int, token: int, pos, cache_pos: int) -> None:
    """Row `row` becomes live: its input token, (t, h, w) positions, cache position,
    and a cleared finished flag.  positions is [3][batch]."""
    token_ids[row] = token
    positions[:, row] = np.asarray(pos, dtype=positions.dtype)
    cache_position[row] = cache_pos
    finished[row] = 0


def slot_retire(finished: np.ndarray, row: int) -> None:
    """Row `row` is finished: the step feeds it the pad id and freezes it."""
    finished[row] = 1
