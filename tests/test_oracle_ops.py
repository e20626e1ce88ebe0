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


# ------------------------------------------------------------------ SiLU and the MLP's gate/up order
# The MLP of a Qwen3 decoder layer is down(silu(gate) * up) with [gate ; up] the rows
# of the fused gate-up projection (kaminari page, section 05: fused gate-up).  SiLU
# is x * sigmoid(x); scipy's expit is an independent sigmoid.

@pytest.mark.parametrize("x", [-40.0, -7.5, -1.0, -1e-3, 0.0, 1e-3, 0.5, 1.0, 3.0, 40.0])
def test_silu_matches_x_times_library_sigmoid(x):
    assert oracle.silu(x) == pytest.approx(x * float(sps.expit(x)), rel=1e-14, abs=1e-300)


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(1.0 / (1.0 + np.exp(-1.0)), rel=1e-15)
    # silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1)
    for x in (0.3, 2.0, 11.0):
        assert oracle.silu(x) - oracle.silu(-x) == pytest.approx(x, rel=1e-14)
    # large |x|: the identity above and the vanishing negative side
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.silu(-40.0)) < 1e-15 and oracle.silu(-40.0) < 0.0


def _mlp_only_layer(dims, rng, gate_std, up_std, zero_gate=False):
    """bf16 source weights of one layer whose O projection is all zero, so that the
    layer's update of x is its MLP alone."""
    H, D, I = dims.hidden, dims.head_dim, dims.intermediate
    bf = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)
    wgu = np.concatenate([rng.standard_normal((I, H)) * gate_std, rng.standard_normal((I, H)) * up_std])
    if zero_gate:
        wgu[:I] = 0.0
    return {
        "in_norm": bf(rng.uniform(0.5, 1.5, H)), "q_norm": bf(rng.uniform(0.5, 1.5, D)),
        "k_norm": bf(rng.uniform(0.5, 1.5, D)), "post_norm": bf(rng.uniform(0.5, 1.5, H)),
        "wqkv": bf(rng.standard_normal((dims.qkv_rows, H)) * 0.02),
        "wo": bf(np.zeros((H, dims.n_heads * D))),
        "wgu": bf(wgu), "wd": bf(rng.standard_normal((H, I)) * 0.02),
    }


@pytest.mark.parametrize("zero_gate", [False, True])
def test_layer_mlp_is_down_of_silu_gate_times_up(zero_gate):
    """Through the oracle's whole layer: x_out - x_in = Wd (silu(g) * u) with
    [g ; u] = Wgu RMSNorm(x_in; post_norm), from the dequantized weights (pinned by
    the quantizer tests) and scipy's sigmoid.  Gate rows are drawn larger than up
    rows, so that silu applied to the up half, or the halves swapped, fails; with
    the gate rows zero the MLP adds exactly nothing."""
    from int4_weight_only_gemv_amd import synth
    dims = synth.TINY
    rng = np.random.default_rng(404)
    w = _mlp_only_layer(dims, rng, 0.2, 0.05, zero_gate)
    model = oracle.Model(dims, [w])
    q = model.q[0]
    B, M = 2, 8
    kc = np.zeros((1, B, dims.n_kv_heads, M, dims.head_dim), np.uint16)
    vc = np.zeros_like(kc)
    x_in = rng.standard_normal((B, dims.hidden)) * 3.0
    x = x_in.copy()
    model.decode_layer(0, kc, vc, x, np.zeros((3, B), np.int32), np.array([2, 5], np.int32))
    G, I = dims.group_size, dims.intermediate
    wgu = oracle.dequant(*q["wgu"], G)
    wd = oracle.dequant(*q["wd"], G)
    for b in range(B):
        h = oracle.rmsnorm(x_in[b], q["post_norm"], dims.rms_eps)
        gu = wgu @ h
        g, u = gu[:I], gu[I:]
        want = wd @ (g * sps.expit(g) * u)
        got = x[b] - x_in[b]
        if zero_gate:
            assert np.all(got == 0.0)
        else:
            assert np.max(np.abs(g)) > 2.0     # the nonlinearity is exercised
            np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12 * np.abs(want).max())
            swapped = wd @ (u * sps.expit(u) * g)
            assert np.abs(swapped - want).max() > 1e-3 * np.abs(want).max()
