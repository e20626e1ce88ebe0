"""GPU parity of kmr_prefill, through the C ABI, against the oracle (kaminari page,
section 04: the prompt's forward fills the static cache; the first generated token
is the argmax at the last prompt token).

- From an empty sequence (start 0) the last token's logits and the written K/V
  slots match the oracle's matrix-form causal forward (oracle/prefill.py).
- After an earlier part of the sequence (start > 0) they match the oracle's own
  decode step run token by token over the same cache row, which is the same
  computation by the decode/prefill invariant.
- Token counts cover one token, a single chunk (group size 128: the matrix-core
  GEMM tiles, ragged; group size 64: the decode path's GEMV tiles), and, with a
  workspace sized for 128 tokens, two chunks with a ragged last one.
- Only the prompt's slots of the chosen cache row change."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle import prefill
from int4_weight_only_gemv_amd import synth
from tests.gpu_util import MARGIN, TOL, bf16_host, build_pair, log, make_caches, max_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kmr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_weight_only_gemv_amd import kmr as m
    return m


@pytest.fixture(scope="module", params=[64, 128], ids=["g64", "g128"])
def pair(kmr, request):
    w = synth.WORKLOADS["kv8"]
    dims = dataclasses.replace(w.dims, group_size=request.param)
    return build_pair(dims, synth.base_seed(w) + request.param, "host", with_globals=True)


def _np_layers(ora):
    return [{k: q[k] for k in ("in_norm", "q_norm", "k_norm", "post_norm", "wqkv", "wo", "wgu", "wd")}
            for q in ora.q]


def _run(kmr, pair, kv, row, tokens, pos3, start, chunk=None):
    dims = pair.dims
    T = len(tokens)
    ws = kmr.Workspace.for_prefill(pair.dev.cfg, chunk or T, kv.k.shape[3])
    nxt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    logits = torch.empty(dims.vocab, dtype=torch.float32, device="cuda")
    pair.dev.prefill(kv, row, torch.from_numpy(tokens.astype(np.int32)).cuda(),
                     torch.from_numpy(np.ascontiguousarray(pos3, np.int32)).cuda(), start, nxt, ws, logits=logits)
    torch.cuda.synchronize()
    assert ws.status() == 0
    return int(nxt.cpu()[0]), logits.cpu().numpy()


def _check_token(got_next, want_logits):
    top = np.sort(want_logits)[-2:]
    if top[1] - top[0] > MARGIN:
        assert got_next == int(np.argmax(want_logits))


def _check_cache(kv, kh, vh, row, lo, hi, want_k, want_v):
    """Row `row` slots [lo, hi) hold want_k/want_v ([L][Hkv][hi-lo][D] bf16 bits) within
    TOL; every other slot of every row keeps its bytes."""
    for dev_t, before, want in ((kv.k, kh, want_k), (kv.v, vh, want_v)):
        got = oracle.as_u16(dev_t)
        changed = np.any(got != before, axis=-1)           # [L][B][Hkv][M]
        ls, bs, gs, ms = np.nonzero(changed)
        assert np.all(bs == row) and np.all((ms >= lo) & (ms < hi))
        err = max_rel(bf16_host(got[:, row, :, lo:hi]).reshape(-1, got.shape[-1]),
                      bf16_host(want).reshape(-1, got.shape[-1]))
        assert err <= TOL, f"K/V max_rel {err:.3e}"


@pytest.mark.parametrize("T,chunk", [(1, None), (13, None), (150, None), (150, 128)])
def test_prefill_from_empty_matches_causal_forward(kmr, pair, T, chunk):
    dims = pair.dims
    w = synth.WORKLOADS["kv8"]
    rng = np.random.default_rng(T)
    tokens = rng.integers(0, dims.vocab, T)
    pos3 = np.sort(rng.integers(0, 300, size=(3, T)), axis=1).astype(np.int32)
    log(f"prefill {T} tokens from position 0 into cache row 1 (group size {dims.group_size}, "
        f"workspace for {chunk or T} tokens)")
    kv, kh, vh = make_caches(dims, synth.base_seed(w) + T, 2, w.max_len, "host")
    got_next, got_logits = _run(kmr, pair, kv, 1, tokens, pos3, 0, chunk)

    x0 = prefill.bf16_values(pair.ora.g["embed"][tokens])
    x_full, kvs = prefill.forward(dims, _np_layers(pair.ora), x0, pos3)
    want = prefill.logits(dims, x_full[-1:], pair.ora.g["final_norm"], pair.ora.g["lm_head"])[0]
    err = max_rel(got_logits[None], want[None])
    log(f"  logits max_rel={err:.3e} next={got_next} oracle argmax={int(np.argmax(want))}")
    assert err <= TOL
    _check_token(got_next, want)
    want_k = np.stack([prefill.to_bf16_bits(kb.transpose(1, 0, 2)) for kb, _ in kvs])   # [L][Hkv][T][D]
    want_v = np.stack([prefill.to_bf16_bits(vb.transpose(1, 0, 2)) for _, vb in kvs])
    _check_cache(kv, kh, vh, 1, 0, T, want_k, want_v)


@pytest.mark.parametrize("start,T", [(100, 20), (127, 66)])
def test_prefill_after_earlier_tokens_matches_decode_steps(kmr, pair, start, T):
    dims = pair.dims
    w = synth.WORKLOADS["kv8"]
    rng = np.random.default_rng(start + T)
    tokens = rng.integers(0, dims.vocab, T)
    pos3 = (start + np.arange(T))[None].repeat(3, 0).astype(np.int32) - np.array([[0], [40], [80]], np.int32)
    log(f"prefill {T} tokens at cache positions {start}..{start + T - 1} of row 0 "
        f"(group size {dims.group_size})")
    kv, kh, vh = make_caches(dims, synth.base_seed(w) + start, 2, w.max_len, "host")
    got_next, got_logits = _run(kmr, pair, kv, 0, tokens, pos3, start)

    kc, vc = kh[:, 0:1].copy(), vh[:, 0:1].copy()
    for t in range(T):
        ref = pair.ora.decode_step(kc, vc, np.array([tokens[t]], np.int32), np.ascontiguousarray(pos3[:, t:t + 1]),
                                   np.array([start + t], np.int32))
    want = ref["logits"][0]
    err = max_rel(got_logits[None], want[None])
    log(f"  logits max_rel={err:.3e} next={got_next} oracle={int(ref['next'][0])} margin={float(ref['margin'][0]):.4f}")
    assert err <= TOL
    if ref["margin"][0] > MARGIN:
        assert got_next == int(ref["next"][0])
    _check_cache(kv, kh, vh, 0, start, start + T, kc[:, 0, :, start:start + T], vc[:, 0, :, start:start + T])


def test_prefill_then_decode_continues_the_sequence(kmr, pair):
    """The cache a prefill leaves is the one the decode step extends: prefill of
    tokens 0..T-2 then one decode step of token T-1 equals the oracle's forward
    over tokens 0..T-1 (the decode/prefill invariant on the device)."""
    dims = pair.dims
    w = synth.WORKLOADS["kv8"]
    T = 40
    rng = np.random.default_rng(7)
    tokens = rng.integers(0, dims.vocab, T)
    pos3 = np.arange(T)[None].repeat(3, 0).astype(np.int32)
    kv, _, _ = make_caches(dims, synth.base_seed(w) + 7, 1, w.max_len, "host")
    _run(kmr, pair, kv, 0, tokens[:-1], pos3[:, :-1], 0)
    ws = kmr.Workspace(pair.dev.cfg, 1, w.max_len)
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty((1, dims.vocab), dtype=torch.float32, device="cuda")
    pair.dev.decode_step(kv, torch.from_numpy(tokens[-1:].astype(np.int32)).cuda(),
                         torch.from_numpy(np.ascontiguousarray(pos3[:, -1:])).cuda(),
                         torch.tensor([T - 1], dtype=torch.int32, device="cuda"), nxt, ws, logits=logits)
    torch.cuda.synchronize()
    assert ws.status() == 0
    x0 = prefill.bf16_values(pair.ora.g["embed"][tokens])
    x_full, _ = prefill.forward(dims, _np_layers(pair.ora), x0, pos3)
    want = prefill.logits(dims, x_full[-1:], pair.ora.g["final_norm"], pair.ora.g["lm_head"])[0]
    err = max_rel(logits.cpu().numpy(), want[None])
    log(f"prefill of {T - 1} tokens, then one decode step: logits max_rel={err:.3e}")
    assert err <= TOL
    _check_token(int(nxt.cpu()[0]), want)


@pytest.mark.parametrize("heads,kv_heads,head_dim", [(16, 4, 64), (8, 8, 128), (8, 2, 128)],
                         ids=["qpg4-d64", "qpg1-d128", "qpg4-d128"])
def test_prefill_gqa_shapes_match_causal_forward(kmr, heads, kv_heads, head_dim):
    """The prefill attention's other GQA group sizes (1 and 4 q heads per kv head: one
    and four waves per group, four and two groups) and head_dim 128 at the reduced
    width, 150 tokens from position 0 in two chunks (workspace for 128 tokens), against
    the oracle's causal forward: last-token logits and every written K/V slot."""
    w = synth.WORKLOADS["kv8"]
    sec = (12, 10, 10) if head_dim == 64 else (24, 20, 20)
    dims = dataclasses.replace(w.dims, n_heads=heads, n_kv_heads=kv_heads, head_dim=head_dim, group_size=128,
                               mrope_section=sec)
    pair = build_pair(dims, synth.base_seed(w) + heads * 100 + kv_heads, "host", with_globals=True)
    T = 150
    rng = np.random.default_rng(heads + kv_heads)
    tokens = rng.integers(0, dims.vocab, T)
    pos3 = np.sort(rng.integers(0, 300, size=(3, T)), axis=1).astype(np.int32)
    log(f"prefill {T} tokens, {heads} q heads / {kv_heads} kv heads of {head_dim}, chunks of 128")
    kv, kh, vh = make_caches(dims, synth.base_seed(w) + T, 2, w.max_len, "host")
    got_next, got_logits = _run(kmr, pair, kv, 1, tokens, pos3, 0, 128)
    x0 = prefill.bf16_values(pair.ora.g["embed"][tokens])
    x_full, kvs = prefill.forward(dims, _np_layers(pair.ora), x0, pos3)
    want = prefill.logits(dims, x_full[-1:], pair.ora.g["final_norm"], pair.ora.g["lm_head"])[0]
    err = max_rel(got_logits[None], want[None])
    log(f"  logits max_rel={err:.3e} next={got_next} oracle argmax={int(np.argmax(want))}")
    assert err <= TOL
    _check_token(got_next, want)
    want_k = np.stack([prefill.to_bf16_bits(kb.transpose(1, 0, 2)) for kb, _ in kvs])
    want_v = np.stack([prefill.to_bf16_bits(vb.transpose(1, 0, 2)) for _, vb in kvs])
    _check_cache(kv, kh, vh, 1, 0, T, want_k, want_v)
