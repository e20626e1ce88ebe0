"""Pins for the oracle's int4 quantizer and int4 matrix-vector product.

The pages (kaminari, section 07) say only that decoder linears become weight-only
int4 with group scales.  The oracle's reading (asymmetric affine codes, zero at
mid-code 8, bf16 scale/zero, ties to even) is pinned here against facts that do
not depend on its own code: the rounding error bound of an affine grid, exact
round trips of on-grid data, a brute-force nearest-code search, exact ties, the
degenerate group, and the independence of rows.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return oracle.as_u16(torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16))


def bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Codes per the layout definition: byte j of a row holds k=2j (low nibble) and k=2j+1."""
    lo = packed & 0x0F
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(packed.shape[0], -1).astype(np.int64)


def dense_from_format(packed, sz, G):
    q = unpack_codes(packed)
    s = np.repeat(bits_to_f32(sz[..., 0]).astype(np.float64), G, axis=1)
    z = np.repeat(bits_to_f32(sz[..., 1]).astype(np.float64), G, axis=1)
    return q, s, z, (q - 8) * s + z


def random_weights(N, K, std=0.02, seed=0):
    r = np.random.default_rng(seed)
    return bf16_bits(r.standard_normal((N, K)).astype(np.float32) * std)


@pytest.mark.parametrize("N,K,G", [(8, 256, 64), (16, 512, 128), (5, 96, 32), (3, 6, 2)])
def test_dequant_matches_layout_definition(N, K, G):
    w = random_weights(N, K, seed=N + K)
    packed, sz = oracle.quantize_int4(w, G)
    _, _, _, dense = dense_from_format(packed, sz, G)
    assert np.array_equal(oracle.dequant(packed, sz, G), dense)


@pytest.mark.parametrize("std", [0.02, 1.0, 300.0])
def test_roundtrip_error_bound(std):
    N, K, G = 64, 512, 128
    w = random_weights(N, K, std=std, seed=7)
    wf = bits_to_f32(w).astype(np.float64)
    packed, sz = oracle.quantize_int4(w, G)
    q, s, z, dense = dense_from_format(packed, sz, G)
    err = np.abs(dense - wf)
    grp = wf.reshape(N, K // G, G)
    rng_ = np.repeat(grp.max(-1) - grp.min(-1), G, axis=1)
    inside = (wf >= z - 8 * s) & (wf <= z + 7 * s)
    # inside the grid the nearest code is within half a step
    assert np.all(err[inside] <= 0.5 * s[inside] * (1 + 1e-5))
    # at the ends the only extra error comes from bf16 rounding of scale and zero
    loose = 0.5 * s * (1 + 1e-5) + rng_ * 2.0**-8 * 1.01 + np.abs(z) * 2.0**-8
    assert np.all(err <= loose)
    assert inside.mean() > 0.95


def test_codes_are_brute_force_nearest_with_ties_to_even():
    N, K, G = 32, 256, 64
    w = random_weights(N, K, seed=3)
    packed, sz = oracle.quantize_int4(w, G)
    q = unpack_codes(packed)
    s32 = np.repeat(bits_to_f32(sz[..., 0]), G, axis=1)
    z32 = np.repeat(bits_to_f32(sz[..., 1]), G, axis=1)
    t = ((bits_to_f32(w) - z32) / s32).astype(np.float32).astype(np.float64)   # binary32 steps
    cand = np.arange(16)[None, None, :] - 8.0
    dist = np.abs(t[..., None] - cand)
    best = dist.min(-1, keepdims=True)
    ties = (dist == best)
    # among equally near codes prefer the even one (round half to even)
    pick = np.where(ties & (np.arange(16) % 2 == 0), 0, 1) + np.where(ties, 0, 2)
    assert np.array_equal(q, np.argmin(pick, axis=-1))


def test_exact_ties_round_to_even():
    # lo = 0, hi = 15/64: scale 1/64 and zero 1/8 are exact; w = (j + 1/2)/64 lies
    # exactly half-way between codes j and j+1.
    G = 32
    vals = [0.0, 15 / 64] + [(j + 0.5) / 64 for j in range(15)]
    vals += [0.0] * (G - len(vals))
    w = bf16_bits(np.array([vals], np.float32))
    packed, sz = oracle.quantize_int4(w, G)
    assert bits_to_f32(sz[0, 0, 0]) == 1 / 64 and bits_to_f32(sz[0, 0, 1]) == 0.125
    q = unpack_codes(packed)[0]
    assert q[0] == 0 and q[1] == 15
    for j in range(15):
        assert q[2 + j] == (j if j % 2 == 0 else j + 1)


@pytest.mark.parametrize("lo,step", [(-1.0, 1 / 16), (3.0, 1 / 8), (-0.03125, 2.0**-10)])
def test_on_grid_group_roundtrips_exactly(lo, step):
    G = 64
    r = np.random.default_rng(11)
    ks = np.concatenate([[0, 15], r.integers(0, 16, size=G - 2)])
    vals = (lo + ks * step).astype(np.float32)
    w = bf16_bits(vals[None, :])
    assert np.array_equal(bits_to_f32(w)[0], vals)          # the grid itself is bf16-exact
    packed, sz = oracle.quantize_int4(w, G)
    assert np.array_equal(oracle.dequant(packed, sz, G)[0], vals.astype(np.float64))
    assert bits_to_f32(sz[0, 0, 0]) == step


@pytest.mark.parametrize("value", [0.0, 0.37109375, -2.5, 1e-3])
def test_degenerate_group(value):
    G = 128
    w = bf16_bits(np.full((1, G), value, np.float32))
    v = bits_to_f32(w)[0, 0]
    packed, sz = oracle.quantize_int4(w, G)
    assert bits_to_f32(sz[0, 0, 0]) == np.float32(2.0**-24)
    deq = oracle.dequant(packed, sz, G)[0]
    assert np.all(np.abs(deq - v) <= max(abs(v) * 2.0**-8, 2.0**-21))


def test_fused_rows_equal_separate_quantization():
    a, b, c = random_weights(24, 256, seed=1), random_weights(8, 256, seed=2), random_weights(8, 256, seed=3)
    pf, sf = oracle.quantize_int4(np.vstack([a, b, c]), 64)
    parts = [oracle.quantize_int4(x, 64) for x in (a, b, c)]
    assert np.array_equal(pf, np.vstack([p for p, _ in parts]))
    assert np.array_equal(sf, np.vstack([s for _, s in parts]))


def test_ieee_fp32_fixture_is_binary32():
    """The Ghost in the Batch prints (a+b)+c for a=1e-7, b=1, c=-1; its value is the
    binary32 result, which is what the brute-force quantizer pin above relies on."""
    g = json.load(open(os.path.join(HERE, "golden", "ieee_fp32_nonassoc.json")))
    a, b, c = np.float32(g["a"]), np.float32(g["b"]), np.float32(g["c"])
    assert float((a + b) + c) == g["left_assoc_printed"]
    assert repr(float(a + (b + c))) != repr(g["left_assoc_printed"])
    assert float(np.float32(g["right_assoc_printed"])) == float(a + (b + c))
    assert (g["a"] + g["b"]) + g["c"] != g["left_assoc_printed"]   # not the binary64 result


# ------------------------------------------------------------------ int4 GEMV

@pytest.mark.parametrize("N,K,G", [(48, 256, 64), (33, 512, 128)])
def test_gemv_one_hot_extracts_columns(N, K, G):
    w = random_weights(N, K, seed=5)
    packed, sz = oracle.quantize_int4(w, G)
    _, _, _, dense = dense_from_format(packed, sz, G)
    ks = [0, 1, G - 1, G, K - 1, K // 2 + 3]
    x = np.zeros((len(ks), K))
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = oracle.gemv_int4(packed, sz, G, x)
    for i, k in enumerate(ks):
        assert np.array_equal(y[i], dense[:, k])


def test_gemv_ones_closed_form():
    N, K, G = 40, 384, 128
    w = random_weights(N, K, seed=9)
    packed, sz = oracle.quantize_int4(w, G)
    q = unpack_codes(packed).reshape(N, K // G, G)
    s = bits_to_f32(sz[..., 0]).astype(np.float64)
    z = bits_to_f32(sz[..., 1]).astype(np.float64)
    expect = (s * (q - 8).sum(-1) + G * z).sum(-1)
    y = oracle.gemv_int4(packed, sz, G, np.ones((1, K)))[0]
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-12)


def test_gemv_within_quantization_error_of_source_weights():
    N, K, G, B = 64, 512, 128, 3
    w = random_weights(N, K, seed=12)
    wf = bits_to_f32(w).astype(np.float64)
    packed, sz = oracle.quantize_int4(w, G)
    q, s, z, dense = dense_from_format(packed, sz, G)
    x = np.random.default_rng(4).standard_normal((B, K))
    y = oracle.gemv_int4(packed, sz, G, x)
    grp = wf.reshape(N, K // G, G)
    rng_ = np.repeat(grp.max(-1) - grp.min(-1), G, axis=1)
    bound = 0.5 * s * (1 + 1e-5) + rng_ * 2.0**-8 * 1.01 + np.abs(z) * 2.0**-8
    assert np.all(np.abs(y - x @ wf.T) <= np.abs(x) @ bound.T + 1e-12)
    np.testing.assert_allclose(y, x @ dense.T, rtol=1e-11, atol=1e-12)


def test_scale_narrowing_ties_to_even():
    # lo = -15/256 and hi = 15 are bf16-exact; (hi - lo) / 15 = 1 + 2^-8 exactly in
    # binary32, half-way between the bf16 values 1 and 1 + 2^-7: ties-to-even gives 1.
    G = 64
    vals = np.linspace(-15 / 256, 15, G).astype(np.float32)
    vals[0], vals[-1] = -15 / 256, 15.0
    w = bf16_bits(vals[None, :])
    assert bits_to_f32(w)[0, 0] == np.float32(-15 / 256) and bits_to_f32(w)[0, -1] == 15.0
    packed, sz = oracle.quantize_int4(w, G)
    assert bits_to_f32(sz[0, 0, 0]) == 1.0
    # zero = bf16(lo + 8 s) = bf16(7.94140625) = 7.9375 (nearest, not a tie)
    assert bits_to_f32(sz[0, 0, 1]) == 7.9375
