"""Pins for the oracle's assembled decoder layer and greedy decode step.

The assembled step has no closed form; it is pinned compositionally (its parts
are pinned in the other oracle tests) and by the decode/prefill invariant: with
a static cache holding the K/V of tokens 0..t-1 (kaminari, section 04: prefill
fills the cache, decode extends it at cache_position), decoding token t must give
the last row of a full causal forward over tokens 0..t.  The forward is a second,
matrix-form implementation (oracle/prefill.py).  Also pinned: only the slot at
cache_position changes, rows are independent, finished rows are fed and emit the
pad id with a frozen position, and the token is the lowest-index argmax.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle import prefill
from int4_weight_only_gemv_amd import synth

DIMS = dataclasses.replace(synth.TINY, n_layers=2)
SEED = 77


@pytest.fixture(scope="module")
def model():
    layers = [synth.layer_weights(DIMS, SEED, l) for l in range(DIMS.n_layers)]
    glob = synth.model_globals(DIMS, SEED)
    return oracle.Model(DIMS, layers, glob)


def np_layers(m):
    return [{"in_norm": q["in_norm"], "q_norm": q["q_norm"], "k_norm": q["k_norm"],
             "post_norm": q["post_norm"], "wqkv": q["wqkv"], "wo": q["wo"], "wgu": q["wgu"],
             "wd": q["wd"]} for q in m.q]


def noise_cache(B, M, seed):
    r = np.random.default_rng(seed)
    shape = (DIMS.n_layers, B, DIMS.n_kv_heads, M, DIMS.head_dim)
    return (prefill.to_bf16_bits(r.standard_normal(shape)),
            prefill.to_bf16_bits(r.standard_normal(shape)))


@pytest.mark.parametrize("T", [1, 2, 24, 63])
def test_decode_equals_last_row_of_causal_prefill(model, T):
    r = np.random.default_rng(T)
    M = 64
    tokens = r.integers(0, DIMS.vocab, T + 0)
    pos3 = r.integers(0, 200, size=(3, T)).astype(np.int32)
    x0 = prefill.bf16_values(model.g["embed"][tokens])
    x_full, kv = prefill.forward(DIMS, np_layers(model), x0, pos3)
    want_logits = prefill.logits(DIMS, x_full[-1:], model.g["final_norm"], model.g["lm_head"])[0]

    kc, vc = noise_cache(1, M, T)
    for l, (kb, vb) in enumerate(kv):
        kc[l, 0, :, : T - 1, :] = prefill.to_bf16_bits(kb[: T - 1].transpose(1, 0, 2))
        vc[l, 0, :, : T - 1, :] = prefill.to_bf16_bits(vb[: T - 1].transpose(1, 0, 2))
    pos = np.ascontiguousarray(pos3[:, T - 1:T])
    cpos = np.array([T - 1], np.int32)
    out = model.decode_step(kc, vc, [tokens[-1]], pos, cpos)

    np.testing.assert_allclose(out["hidden"][0], x_full[-1], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(out["logits"][0], want_logits, rtol=1e-9, atol=1e-10)
    for l, (kb, vb) in enumerate(kv):
        assert np.array_equal(kc[l, 0, :, T - 1, :], prefill.to_bf16_bits(kb[T - 1]))
        assert np.array_equal(vc[l, 0, :, T - 1, :], prefill.to_bf16_bits(vb[T - 1]))


def test_only_cache_position_slots_change(model):
    B, M = 3, 48
    kc, vc = noise_cache(B, M, 1)
    k0, v0 = kc.copy(), vc.copy()
    cpos = np.array([5, 0, 47], np.int32)
    pos = np.array([[5, 0, 47], [3, 9, 1], [2, 2, 2]], np.int32)
    model.decode_step(kc, vc, [1, 2, 3], pos, cpos)
    mask = np.zeros(kc.shape, bool)
    for b in range(B):
        mask[:, b, :, cpos[b], :] = True
    assert np.array_equal(kc[~mask], k0[~mask]) and np.array_equal(vc[~mask], v0[~mask])
    assert not np.array_equal(kc[mask], k0[mask])


def test_rows_are_independent(model):
    B, M = 3, 40
    kc, vc = noise_cache(B, M, 2)
    ids = np.array([10, 500, 1023], np.int32)
    pos = np.array([[4, 30, 7], [1, 30, 6], [0, 29, 5]], np.int32)
    cpos = np.array([4, 30, 39], np.int32)
    allrows = model.decode_step(kc.copy(), vc.copy(), ids, pos.copy(), cpos.copy())
    for b in range(B):
        one = model.decode_step(np.ascontiguousarray(kc[:, b:b + 1]), np.ascontiguousarray(vc[:, b:b + 1]),
                                ids[b:b + 1], np.ascontiguousarray(pos[:, b:b + 1]), cpos[b:b + 1].copy())
        assert np.array_equal(one["logits"][0], allrows["logits"][b])


def test_argmax_and_margin(model):
    kc, vc = noise_cache(2, 32, 3)
    out = model.decode_step(kc, vc, [7, 8], np.array([[1, 2], [3, 4], [5, 6]], np.int32),
                            np.array([9, 10], np.int32))
    for b in range(2):
        lg = out["logits"][b]
        assert out["next"][b] == int(np.argmax(lg))
        top = np.sort(lg)[::-1]
        assert out["margin"][b] == top[0] - top[1]


def test_finished_rows_and_advance(model):
    B, M = 3, 32
    kc, vc = noise_cache(B, M, 4)
    ids = np.array([11, 12, 13], np.int32)
    pos = np.array([[3, 8, 31], [4, 8, 30], [5, 8, 29]], np.int32)
    cpos = np.array([3, 8, M - 1], np.int32)
    fin = np.array([0, 1, 0], np.uint8)
    ref = model.decode_step(kc.copy(), vc.copy(), np.array([11, DIMS.pad_id, 13], np.int32),
                            pos.copy(), cpos.copy())
    p2, c2 = pos.copy(), cpos.copy()
    out = model.decode_step(kc, vc, ids, p2, c2, finished=fin, advance=True)
    # a finished row is fed the pad id and emits it; its slot is still computed
    assert np.array_equal(out["logits"][1], ref["logits"][1])
    assert out["next"][1] == DIMS.pad_id
    assert out["next"][0] == ref["next"][0] and out["next"][2] == ref["next"][2]
    assert list(c2) == [4, 8, M - 1]
    assert np.array_equal(p2[:, 0], pos[:, 0] + 1) and np.array_equal(p2[:, 1:], pos[:, 1:])
    assert list(fin) == [0, 1, 1]            # row 2 reached the last slot: length stop


def test_eos_finishes_row(model):
    kc, vc = noise_cache(1, 32, 5)
    pos, cpos = np.array([[2], [2], [2]], np.int32), np.array([2], np.int32)
    first = model.decode_step(kc.copy(), vc.copy(), [3], pos.copy(), cpos.copy())
    eos_model = oracle.Model(dataclasses.replace(DIMS, eos_id=int(first["next"][0])), [], None)
    eos_model.q, eos_model.clayers, eos_model.g = model.q, model.clayers, model.g
    eos_model.cmodel = model.cmodel
    fin = np.zeros(1, np.uint8)
    out = eos_model.decode_step(kc, vc, [3], pos, cpos, finished=fin, advance=True)
    assert out["next"][0] == first["next"][0] and fin[0] == 1 and cpos[0] == 2


def test_out_of_range_cache_position_is_rejected(model):
    kc, vc = noise_cache(1, 16, 6)
    k0 = kc.copy()
    with pytest.raises(ValueError):
        model.decode_step(kc, vc, [1], np.zeros((3, 1), np.int32), np.array([16], np.int32))
    assert np.array_equal(kc, k0)
