"""Pins for the oracle's RMSNorm, 3D M-RoPE and attention.

Each check rests on something other than the oracle's own formula: a closed form,
the textbook 1-D rotary embedding (complex rotation), rotation invariants, a
library softmax / logsumexp, or the log-sum-exp merge of partial attentions that
"The Ghost in the Batch" states ("The merge math").
"""
import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle


def bf16_bits(x) -> np.ndarray:
    return oracle.as_u16(torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16))


def bits_to_f64(u) -> np.ndarray:
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ RMSNorm

@pytest.mark.parametrize("c,eps", [(1e-3, 1e-6), (2.0, 1e-6), (-0.5, 0.0), (1e-3, 0.0)])
def test_rmsnorm_constant_vector_closed_form(c, eps):
    n = 256
    gain = bf16_bits(np.random.default_rng(0).uniform(0.5, 1.5, n))
    out = oracle.rmsnorm(np.full(n, c), gain, eps)
    np.testing.assert_allclose(out, c / np.sqrt(c * c + eps) * bits_to_f64(gain), rtol=1e-14)


def test_rmsnorm_two_element_closed_form():
    gain = bf16_bits([1.0, 0.75])
    out = oracle.rmsnorm(np.array([3.0, 4.0]), gain, 1e-6)
    inv = 1.0 / np.sqrt(12.5 + 1e-6)
    np.testing.assert_allclose(out, [3.0 * inv, 4.0 * inv * 0.75], rtol=1e-15)


def test_rmsnorm_scale_invariance_for_large_inputs():
    r = np.random.default_rng(1)
    x = r.standard_normal(512)
    gain = bf16_bits(r.uniform(0.5, 1.5, 512))
    np.testing.assert_allclose(oracle.rmsnorm(1e6 * x, gain, 1e-6), oracle.rmsnorm(x, gain, 0.0),
                               rtol=1e-12)


# ------------------------------------------------------------------ M-RoPE

THETA = 5_000_000.0


def textbook_rope(x, p, theta):
    """1-D rotary embedding, rotate-half form: pair (j, j+D/2) as the complex number
    x_j + i x_{j+D/2}, multiplied by exp(i p theta^(-2j/D))."""
    D = x.shape[-1]
    h = D // 2
    ang = p * theta ** (-2.0 * np.arange(h) / D)
    z = (x[:h] + 1j * x[h:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag])


@pytest.mark.parametrize("D,sec", [(128, (24, 20, 20)), (64, (12, 10, 10))])
@pytest.mark.parametrize("inter", [1, 0])
def test_mrope_axis_counts_equal_sections(D, sec, inter):
    axes = [oracle.mrope_axis(j, D // 2, sec, inter) for j in range(D // 2)]
    assert [axes.count(a) for a in (0, 1, 2)] == list(sec)


def test_mrope_interleaved_and_contiguous_tables():
    sec = (24, 20, 20)
    inter = [oracle.mrope_axis(j, 64, sec, 1) for j in range(64)]
    assert inter[:6] == [0, 1, 2, 0, 1, 2]
    assert inter[57:] == [0, 1, 2, 0, 0, 0, 0]
    cont = [oracle.mrope_axis(j, 64, sec, 0) for j in range(64)]
    assert cont == [0] * 24 + [1] * 20 + [2] * 20


@pytest.mark.parametrize("inter", [1, 0])
def test_mrope_zero_position_is_identity(inter):
    x = np.random.default_rng(2).standard_normal(128)
    assert np.array_equal(oracle.mrope(x, [0, 0, 0], (24, 20, 20), inter, THETA), x)


@pytest.mark.parametrize("inter", [1, 0])
@pytest.mark.parametrize("p", [1, 220, 7999])
def test_mrope_equal_axes_is_textbook_rope(inter, p):
    x = np.random.default_rng(p).standard_normal(128)
    np.testing.assert_allclose(oracle.mrope(x, [p, p, p], (24, 20, 20), inter, THETA),
                               textbook_rope(x, p, THETA), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("inter", [1, 0])
def test_mrope_single_axis_rotates_only_its_pairs(inter):
    sec = (24, 20, 20)
    x = np.random.default_rng(3).standard_normal(128)
    for ax in range(3):
        p = [0, 0, 0]
        p[ax] = 37
        y = oracle.mrope(x, p, sec, inter, THETA)
        full = textbook_rope(x, 37, THETA)
        for j in range(64):
            own = oracle.mrope_axis(j, 64, sec, inter) == ax
            for idx in (j, j + 64):
                if own:
                    assert abs(y[idx] - full[idx]) < 1e-12
                else:
                    assert y[idx] == x[idx]


def test_mrope_preserves_pair_norms_and_is_relative():
    r = np.random.default_rng(4)
    q, k = r.standard_normal(128), r.standard_normal(128)
    pos = np.array([51, 17, 90])
    y = oracle.mrope(q, pos, (24, 20, 20), 1, THETA)
    np.testing.assert_allclose(y[:64] ** 2 + y[64:] ** 2, q[:64] ** 2 + q[64:] ** 2, rtol=1e-12)

    def dot(pq, pk):
        return oracle.mrope(q, [pq] * 3, (24, 20, 20), 1, THETA) @ oracle.mrope(k, [pk] * 3, (24, 20, 20), 1, THETA)
    np.testing.assert_allclose(dot(700, 650), dot(50, 0), rtol=1e-9)
    np.testing.assert_allclose(dot(8000, 10), dot(7990, 0), rtol=1e-9)


# ------------------------------------------------------------------ attention

def rand_kv(n, D, seed):
    r = np.random.default_rng(seed)
    return bf16_bits(r.standard_normal((n, D))), bf16_bits(r.standard_normal((n, D)))


def test_attention_single_position_returns_value_row():
    k, v = rand_kv(1, 64, 0)
    q = np.random.default_rng(1).standard_normal(64) * 10
    assert np.array_equal(oracle.attend(q, k, v), bits_to_f64(v[0]))


def test_attention_equal_keys_average_values():
    k, v = rand_kv(37, 64, 2)
    k[:] = k[0]
    q = np.random.default_rng(3).standard_normal(64)
    np.testing.assert_allclose(oracle.attend(q, k, v), bits_to_f64(v).mean(0), rtol=1e-12, atol=1e-14)


def test_attention_dominant_key_selects_its_value():
    k, v = rand_kv(50, 128, 4)
    kf = bits_to_f64(k)
    q = 400.0 * kf[17] / np.linalg.norm(kf[17])
    np.testing.assert_allclose(oracle.attend(q, k, v), bits_to_f64(v[17]), atol=1e-6)


@pytest.mark.parametrize("n,D", [(1, 64), (5, 64), (129, 128), (700, 128)])
def test_attention_matches_library_softmax(n, D):
    k, v = rand_kv(n, D, n)
    q = np.random.default_rng(n + 1).standard_normal(D) * 2
    p = sps.softmax(bits_to_f64(k) @ q / np.sqrt(D))
    np.testing.assert_allclose(oracle.attend(q, k, v), p @ bits_to_f64(v), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("cuts", [[64], [1, 300], [128, 256, 511]])
def test_attention_lse_merge_of_splits_equals_single_pass(cuts):
    n, D = 600, 128
    k, v = rand_kv(n, D, 9)
    q = np.random.default_rng(10).standard_normal(D) * 3
    s = bits_to_f64(k) @ q / np.sqrt(D)
    bounds = [0] + cuts + [n]
    outs, lses = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        outs.append(oracle.attend(q, k[a:b], v[a:b]))
        lses.append(sps.logsumexp(s[a:b]))
    mx = max(lses)
    wts = np.exp(np.array(lses) - mx)
    merged = (wts[:, None] * np.array(outs)).sum(0) / wts.sum()
    np.testing.assert_allclose(merged, oracle.attend(q, k, v), rtol=1e-12, atol=1e-13)


def test_bf16_rounding_ties_and_neighbours():
    # 1 + 2^-8 is half-way between 1 and 1 + 2^-7: ties go to the even mantissa (1).
    assert oracle.bf16_round(1.0 + 2.0**-8) == 1.0
    assert oracle.bf16_round(1.0 + 3 * 2.0**-8) == 1.0 + 2 * 2.0**-7
    assert oracle.bf16_round(1.0 + 2.0**-8 + 2.0**-40) == 1.0 + 2.0**-7
    assert oracle.bf16_round(-3.0) == -3.0
    r = np.random.default_rng(5).standard_normal(2000)
    ref = torch.from_numpy(r.astype(np.float32)).to(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_round(float(np.float32(x))) for x in r])
    assert np.array_equal(got, ref)
