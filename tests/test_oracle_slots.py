"""Pins for the oracle's slot operations (oracle/slots.py), through the decode
oracle: a row whose cache was copied into another slot of another cache decodes
exactly like the original row, only the copied positions of the destination row
change, an admitted row decodes like a row given the same inputs directly, and a
retired row is fed the pad id and frozen (kaminari, section 08: continuous
batching over per-row cache slots; section 03: the state a live row carries)."""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle import prefill, slots
from int4_weight_only_gemv_amd import synth

DIMS = dataclasses.replace(synth.TINY, n_layers=2)
SEED = 91


@pytest.fixture(scope="module")
def model():
    layers = [synth.layer_weights(DIMS, SEED, l) for l in range(DIMS.n_layers)]
    return oracle.Model(DIMS, layers, synth.model_globals(DIMS, SEED))


def noise_cache(B, M, seed):
    r = np.random.default_rng(seed)
    shape = (DIMS.n_layers, B, DIMS.n_kv_heads, M, DIMS.head_dim)
    return (prefill.to_bf16_bits(r.standard_normal(shape)),
            prefill.to_bf16_bits(r.standard_normal(shape)))


@pytest.mark.parametrize("c", [0, 1, 17, 39])
def test_copied_row_decodes_like_the_original(model, c):
    ka, va = noise_cache(3, 40, 1)
    kb, vb = noise_cache(2, 48, 2)
    slots.kv_copy_row(kb, vb, 0, ka, va, 1, c)
    pos = np.array([[c], [c // 2], [c // 3]], np.int32)
    want = model.decode_step(np.ascontiguousarray(ka[:, 1:2]), np.ascontiguousarray(va[:, 1:2]), [321],
                             pos.copy(), np.array([c], np.int32))
    got = model.decode_step(np.ascontiguousarray(kb[:, 0:1]), np.ascontiguousarray(vb[:, 0:1]), [321],
                            pos.copy(), np.array([c], np.int32))
    assert np.array_equal(got["logits"], want["logits"]) and got["next"][0] == want["next"][0]


def test_copy_changes_only_the_copied_positions(model):
    ka, va = noise_cache(2, 30, 3)
    kb, vb = noise_cache(3, 20, 4)
    k0, v0 = kb.copy(), vb.copy()
    slots.kv_copy_row(kb, vb, 2, ka, va, 0, 13)
    mask = np.zeros(kb.shape, bool)
    mask[:, 2, :, :13, :] = True
    assert np.array_equal(kb[~mask], k0[~mask]) and np.array_equal(vb[~mask], v0[~mask])
    assert np.array_equal(kb[:, 2, :, :13], ka[:, 0, :, :13])
    assert np.array_equal(vb[:, 2, :, :13], va[:, 0, :, :13])
    with pytest.raises(ValueError):
        slots.kv_copy_row(kb, vb, 0, ka, va, 0, 21)


def test_admitted_row_decodes_like_direct_inputs(model):
    kc, vc = noise_cache(2, 32, 5)
    ids = np.array([4, 0], np.int32)
    pos = np.array([[6, 0], [2, 0], [1, 0]], np.int32)
    cpos = np.array([6, 0], np.int32)
    fin = np.array([0, 1], np.uint8)
    slots.slot_admit(ids, pos, cpos, fin, 1, 700, (20, 9, 4), 20)
    assert ids[1] == 700 and list(pos[:, 1]) == [20, 9, 4] and cpos[1] == 20 and fin[1] == 0
    got = model.decode_step(kc.copy(), vc.copy(), ids, pos.copy(), cpos.copy(), finished=fin.copy())
    want = model.decode_step(np.ascontiguousarray(kc[:, 1:2]), np.ascontiguousarray(vc[:, 1:2]), [700],
                             np.array([[20], [9], [4]], np.int32), np.array([20], np.int32))
    assert np.array_equal(got["logits"][1], want["logits"][0])


def test_retired_row_is_fed_pad_and_frozen(model):
    kc, vc = noise_cache(2, 32, 6)
    ids = np.array([5, 9], np.int32)
    pos = np.array([[3, 8], [3, 8], [3, 8]], np.int32)
    cpos = np.array([3, 8], np.int32)
    fin = np.zeros(2, np.uint8)
    slots.slot_retire(fin, 0)
    p2, c2 = pos.copy(), cpos.copy()
    out = model.decode_step(kc, vc, ids, p2, c2, finished=fin, advance=True)
    assert out["next"][0] == DIMS.pad_id
    assert c2[0] == 3 and np.array_equal(p2[:, 0], pos[:, 0])
    assert c2[1] == 9 and np.array_equal(p2[:, 1], pos[:, 1] + 1)
