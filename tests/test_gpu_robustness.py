"""GPU tests of the failure paths and of inputs outside the usual ranges, through
the C ABI against the CPU oracle:

  - a persistent step whose waits give up (forced from the host with the
    KMR_TEST_STALL hook, so every work-group still exits through its bounded
    wait) writes -1 to next_ids, advances nothing, writes no cache slot, raises
    KMR_STATUS_TIMEOUT, and keeps refusing until the workspace is re-initialised
    (kaminari page, section 07: failures are explicit and fail hard);
  - one workspace serves a prefill, a batch-1 decode and a batch-4 decode in turn;
  - residual-stream magnitudes of 1e4..1e5 and MLP activations past the fp16 range
    (the persistent kernel stages them scaled by 2^-3, finite up to about 5.2e5;
    the per-phase kernels, which stage activations unscaled, raise
    KMR_STATUS_RANGE for one they cannot stage);
  - the contiguous M-RoPE section layout with distinct t/h/w positions on every
    kernel path.
Bars as in test_gpu_parity: logits and written K/V within max relative error 2e-2,
tokens equal where the oracle's top-2 margin exceeds 1e-2, other cache bytes equal.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from int4_weight_only_gemv_amd import synth
from tests.gpu_util import MARGIN, TOL, bf16_host, build_pair, log, make_caches, max_rel

pytestmark = pytest.mark.gpu

PATH_FLAGS = {
    "persistent": {},
    "device_scope_stores": {"device_scope_stores": True},
    "device_wide": {"device_wide": True},
    "multi_kernel": {"multi_kernel": True},
}


@pytest.fixture(scope="module")
def kmr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_weight_only_gemv_amd import kmr as k
    return k


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check(got_next, got_logits, ref, label):
    lerr = max_rel(got_logits, ref["logits"])
    decisive = ref["margin"] > MARGIN
    log(f"  {label}: logits max_rel={lerr:.3e} tokens={got_next.tolist()} ref={ref['next'].tolist()}")
    assert lerr <= TOL
    assert np.all((got_next == ref["next"]) | ~decisive)


def _check_cache(kv, kh, vh, written):
    for dev_t, ref in ((kv.k, kh), (kv.v, vh)):
        got = oracle.as_u16(dev_t)
        diff = np.any(got != ref, axis=-1)
        for l, b, g, m in zip(*np.nonzero(diff)):
            assert (int(b), int(m)) in written, f"slot {(l, b, g, m)} changed but was not written"
        for b, m in written:
            err = max_rel(bf16_host(got[:, b, :, m, :]).reshape(-1, got.shape[-1]),
                          bf16_host(ref[:, b, :, m, :]).reshape(-1, got.shape[-1]))
            assert err <= TOL, f"row {b} slot {m}: K/V max_rel {err:.3e}"


def _lockstep(kmr, pair, kv, kh, vh, inp, ws, steps, flags, written=None):
    """`steps` advancing steps, both sides fed the oracle's token; returns the
    slots written."""
    B = len(inp["ids"])
    M = kh.shape[3]
    ids = inp["ids"].copy()
    pos, cpos, fin = inp["positions"].copy(), inp["cache_position"].copy(), inp["finished"].copy()
    pos_d, cpos_d, fin_d = _dev(pos), _dev(cpos), _dev(fin)
    nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, pair.dims.vocab), dtype=torch.float32, device="cuda")
    written = set() if written is None else written
    for s in range(steps):
        written.update((b, int(c)) for b, c in enumerate(cpos) if 0 <= c < M)
        pair.dev.decode_step(kv, _dev(ids), pos_d, cpos_d, nxt, ws, finished=fin_d, logits=logits,
                             advance=True, **flags)
        torch.cuda.synchronize()
        ref = pair.ora.decode_step(kh, vh, ids, pos, cpos, finished=fin, advance=True)
        _check(nxt.cpu().numpy(), logits.cpu().numpy(), ref, f"step {s}")
        assert np.array_equal(pos_d.cpu().numpy(), pos) and np.array_equal(cpos_d.cpu().numpy(), cpos)
        ids = ref["next"].astype(np.int32)
    return written


@pytest.fixture(scope="module")
def kv8_pair(kmr):
    w = synth.WORKLOADS["kv8"]
    return build_pair(w.dims, synth.base_seed(w), "host", with_globals=True)


@pytest.fixture(scope="module")
def tiny_pair(kmr):
    w = synth.WORKLOADS["tiny"]
    return build_pair(w.dims, synth.base_seed(w), "host", with_globals=True)


# ------------------------------------------------------------------ timeouts

def stall_then_recover(kmr, pair, w, flags, batch=None, inp=None):
    """A stalled step (KMR_TEST_STALL), a refused plain step, then a re-initialised
    workspace that decodes like the oracle."""
    inp = synth.step_inputs(w) if inp is None else inp
    B = len(inp["ids"]) if batch is None else batch
    inp = {k: np.ascontiguousarray(v[..., :B]) for k, v in inp.items()}
    kv, kh, vh = make_caches(pair.dims, synth.base_seed(w), B, w.max_len,
                             "host" if pair.dims.n_layers <= 2 else "device")
    k0, v0 = kv.k.clone(), kv.v.clone()
    ws = kmr.Workspace(pair.dev.cfg, B, w.max_len)
    pos_d, cpos_d, fin_d = _dev(inp["positions"]), _dev(inp["cache_position"]), _dev(inp["finished"])
    nxt = torch.full((B,), 7, dtype=torch.int32, device="cuda")
    for extra, label in ((kmr.KMR_TEST_STALL, "stalled"), (0, "refused")):
        nxt.fill_(7)
        pair.dev.decode_step(kv, _dev(inp["ids"]), pos_d, cpos_d, nxt, ws, finished=fin_d, advance=True,
                             extra_flags=extra, **flags)
        torch.cuda.synchronize()
        st = ws.status()
        log(f"  {label} step: next={nxt.cpu().tolist()} status={st}")
        assert torch.all(nxt == -1)
        assert st & kmr.KMR_STATUS_TIMEOUT
        assert np.array_equal(pos_d.cpu().numpy(), inp["positions"])
        assert np.array_equal(cpos_d.cpu().numpy(), inp["cache_position"])
        assert np.array_equal(fin_d.cpu().numpy(), inp["finished"])
        assert torch.equal(kv.k, k0) and torch.equal(kv.v, v0)
    ws.init()
    assert ws.status() == 0
    written = _lockstep(kmr, pair, kv, kh, vh, inp, ws, 2, flags)
    assert ws.status() == 0
    _check_cache(kv, kh, vh, written)


@pytest.mark.parametrize("path", ["persistent", "device_scope_stores", "device_wide"])
def test_stalled_step_fails_hard_then_recovers_kv8(kmr, kv8_pair, path):
    log(f"kv8 batch 4: stalled persistent step, refusal, re-initialised workspace ({path})")
    stall_then_recover(kmr, kv8_pair, synth.WORKLOADS["kv8"], PATH_FLAGS[path])


def test_stalled_step_fails_hard_then_recovers_batch1(kmr, kv8_pair):
    log("kv8 batch 1: stalled persistent step, refusal, re-initialised workspace")
    stall_then_recover(kmr, kv8_pair, synth.WORKLOADS["kv8"], {}, batch=1)


def test_stalled_step_fails_hard_then_recovers_tiny(kmr, tiny_pair):
    """The tiny model has 2 kv heads: its default persistent kernel is the device-wide one."""
    log("tiny batch 1: stalled persistent step, refusal, re-initialised workspace")
    stall_then_recover(kmr, tiny_pair, synth.WORKLOADS["tiny"], {})


# ------------------------------------------------------------------ one workspace, every call kind

def test_workspace_serves_prefill_then_batch1_then_batch4(kmr, kv8_pair):
    """A 13-token prefill of row 0, a batch-1 step of row 0 and two batch-4 steps,
    all on one workspace (sized for the largest of them) and one batch-4 cache."""
    pair = kv8_pair
    w = synth.WORKLOADS["kv8"]
    dims, M, T = pair.dims, w.max_len, 13
    log("kv8: prefill 13 tokens, then batch-1 and batch-4 decode steps on one workspace")
    nbytes = max(kmr.workspace_bytes(pair.dev.cfg, 4, M), kmr.workspace_bytes(pair.dev.cfg, 1, M),
                 kmr.prefill_workspace_bytes(pair.dev.cfg, T, M))
    ws = kmr.Workspace(pair.dev.cfg, 0, M, nbytes=nbytes)
    kv, kh, vh = make_caches(dims, synth.base_seed(w) + 77, 4, M, "host")
    rng = np.random.default_rng(1313)
    tokens = rng.integers(0, dims.vocab, T).astype(np.int32)
    pos3 = np.ascontiguousarray(np.stack([np.arange(T), np.arange(T) // 2, np.arange(T) // 3]).astype(np.int32))
    nxt1 = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    logits1 = torch.empty(dims.vocab, dtype=torch.float32, device="cuda")
    pair.dev.prefill(kv, 0, _dev(tokens), _dev(pos3), 0, nxt1, ws, logits=logits1)
    torch.cuda.synchronize()
    assert ws.status() == 0
    # the oracle: the prompt token by token through its decode step on row 0
    k0, v0 = np.ascontiguousarray(kh[:, 0:1]), np.ascontiguousarray(vh[:, 0:1])
    for t in range(T):
        ref = pair.ora.decode_step(k0, v0, tokens[t:t + 1], np.ascontiguousarray(pos3[:, t:t + 1]),
                                   np.array([t], np.int32))
    _check(nxt1.cpu().numpy(), logits1.cpu().numpy()[None], ref, "prefill")
    written = {(0, t) for t in range(T)}
    # batch 1 on row 0 of the batch-4 cache
    inp1 = {"ids": ref["next"].astype(np.int32), "positions": np.array([[T], [T // 2 + 1], [T // 3 + 1]], np.int32),
            "cache_position": np.array([T], np.int32), "finished": np.zeros(1, np.uint8)}
    _lockstep(kmr, pair, kv, k0, v0, inp1, ws, 1, {}, written)
    kh[:, 0:1], vh[:, 0:1] = k0, v0
    # batch 4 over all rows
    inp4 = synth.step_inputs(w)
    inp4["cache_position"][0] = T + 1
    inp4["positions"][:, 0] = [T + 1, T // 2 + 2, T // 3 + 2]
    _lockstep(kmr, pair, kv, kh, vh, inp4, ws, 2, {}, written)
    assert ws.status() == 0
    _check_cache(kv, kh, vh, written)


# ------------------------------------------------------------------ magnitudes

OUTLIERS = {3: 6.0e4, 100: -1.0e5, 257: 3.1e4, 500: 1.2e5, 511: -4.4e4}


def _outlier_pair(dims, seed, scale_gate_up=None):
    """kv8-shaped model whose embedding rows carry residual outliers of 3e4..1.2e5 in
    fixed channels (and, optionally, layer 0's gate/up weights scaled up)."""
    layers = [synth.layer_weights(dims, seed, l) for l in range(dims.n_layers)]
    if scale_gate_up is not None:
        layers[0]["wgu"] = (layers[0]["wgu"].float() * scale_gate_up).to(torch.bfloat16)
    glob = synth.model_globals(dims, seed)
    for ch, val in OUTLIERS.items():
        glob["embed"][:, ch] = val
    from int4_weight_only_gemv_amd import kmr
    dev = kmr.DeviceModel(dims, layers, glob)
    ora = oracle.Model(dims, [{k: oracle.as_u16(v) for k, v in l.items()} for l in layers],
                       {k: oracle.as_u16(v) for k, v in glob.items()})
    from tests.gpu_util import Pair
    return Pair(dims, dev, ora)


@pytest.mark.parametrize("path", ["persistent", "device_scope_stores", "device_wide", "multi_kernel"])
def test_residual_outliers_1e5_step(kmr, path):
    w = synth.WORKLOADS["kv8"]
    log(f"kv8 batch 4: residual stream with outlier channels up to 1.2e5, 2 steps ({path})")
    pair = _outlier_pair(w.dims, synth.base_seed(w))
    kv, kh, vh = make_caches(w.dims, synth.base_seed(w), w.batch, w.max_len, "host")
    ws = kmr.Workspace(pair.dev.cfg, w.batch, w.max_len)
    written = _lockstep(kmr, pair, kv, kh, vh, synth.step_inputs(w), ws, 2, PATH_FLAGS[path])
    assert ws.status() == 0
    _check_cache(kv, kh, vh, written)


def test_residual_outliers_1e5_layer(kmr):
    """kmr_decode_layer (per-phase kernels) on a residual with channels of 1e4..1e5."""
    w = synth.WORKLOADS["kv8"]
    log("kv8 decode_layer, batch 3, residual outliers 1e4..1e5")
    pair = build_pair(w.dims, synth.base_seed(w), "host", with_globals=False)
    kv, kh, vh = make_caches(w.dims, synth.base_seed(w), 3, w.max_len, "host")
    x0 = synth.hidden_input(w.dims, 31, 3).numpy().copy()
    x0[:, [7, 64, 300]] = [[1e4, -5e4, 1e5], [-1e5, 2e4, 3e4], [6.5e4, -6.5e4, 1.5e4]]
    cpos = np.array([5, 200, 383], np.int32)
    pos = np.array([[5, 200, 383], [1, 7, 9], [2, 2, 300]], np.int32)
    ws = kmr.Workspace(pair.dev.cfg, 3, w.max_len)
    x_dev = torch.from_numpy(x0.astype(np.float32)).cuda()
    pair.dev.decode_layer(0, kv, x_dev, _dev(pos), _dev(cpos), ws)
    torch.cuda.synchronize()
    assert ws.status() == 0
    x_ref = x0.astype(np.float64).copy()
    pair.ora.decode_layer(0, kh, vh, x_ref, pos, cpos)
    err = max_rel(x_dev.cpu().numpy(), x_ref)
    log(f"  hidden max_rel={err:.3e}")
    assert err <= TOL
    _check_cache(kv, kh, vh, {(b, int(c)) for b, c in enumerate(cpos)})


def test_mlp_activation_past_fp16_range(kmr):
    """Layer 0's gate/up weights scaled by 250 (with the residual outliers above)
    drive SiLU(gate)*up past 65504 for some channels, to about 1.3e5.  The persistent
    kernel stages the activations scaled by 2^-3 and matches the oracle; the
    per-phase kernels cannot stage them and say so with KMR_STATUS_RANGE."""
    w = synth.WORKLOADS["kv8"]
    log("kv8 batch 4: MLP activations past 65504 (gate/up weights x250)")
    pair = _outlier_pair(w.dims, synth.base_seed(w), scale_gate_up=250.0)
    kv, kh, vh = make_caches(w.dims, synth.base_seed(w), w.batch, w.max_len, "host")
    ws = kmr.Workspace(pair.dev.cfg, w.batch, w.max_len)
    _lockstep(kmr, pair, kv, kh, vh, synth.step_inputs(w), ws, 1, {})
    assert ws.status() == 0
    kv2, _, _ = make_caches(w.dims, synth.base_seed(w), w.batch, w.max_len, "host", host_rows=[])
    inp = synth.step_inputs(w)
    nxt = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    pair.dev.decode_step(kv2, _dev(inp["ids"]), _dev(inp["positions"]), _dev(inp["cache_position"]), nxt, ws,
                         multi_kernel=True)
    assert ws.status() & kmr.KMR_STATUS_RANGE


# ------------------------------------------------------------------ M-RoPE layout

@pytest.mark.parametrize("path", ["persistent", "device_wide", "multi_kernel"])
def test_contiguous_mrope_sections(kmr, path):
    """mrope_interleaved = 0 (contiguous t | h | w blocks of frequency pairs) with
    distinct t, h, w positions in every row."""
    w = synth.WORKLOADS["kv8"]
    dims = dataclasses.replace(w.dims, mrope_interleaved=0)
    log(f"kv8 batch 4, contiguous M-RoPE sections, distinct t/h/w, 3 steps ({path})")
    pair = build_pair(dims, synth.base_seed(w), "host", with_globals=True)
    kv, kh, vh = make_caches(dims, synth.base_seed(w), w.batch, w.max_len, "host")
    inp = synth.step_inputs(w)
    inp["positions"] = np.ascontiguousarray(np.stack([inp["cache_position"], inp["cache_position"] // 2 + 3,
                                                      inp["cache_position"] // 3 + 11]).astype(np.int32))
    ws = kmr.Workspace(pair.dev.cfg, w.batch, w.max_len)
    written = _lockstep(kmr, pair, kv, kh, vh, inp, ws, 3, PATH_FLAGS[path])
    assert ws.status() == 0
    _check_cache(kv, kh, vh, written)


def test_contiguous_mrope_layer(kmr):
    w = synth.WORKLOADS["kv8"]
    dims = dataclasses.replace(w.dims, mrope_interleaved=0)
    log("kv8 decode_layer, contiguous M-RoPE sections, batch 2")
    pair = build_pair(dims, synth.base_seed(w), "host", with_globals=False)
    kv, kh, vh = make_caches(dims, synth.base_seed(w), 2, w.max_len, "host")
    x0 = synth.hidden_input(dims, 12, 2).numpy()
    cpos = np.array([40, 300], np.int32)
    pos = np.array([[40, 300], [9, 120], [33, 2]], np.int32)
    ws = kmr.Workspace(pair.dev.cfg, 2, w.max_len)
    x_dev = torch.from_numpy(x0.astype(np.float32)).cuda()
    pair.dev.decode_layer(0, kv, x_dev, _dev(pos), _dev(cpos), ws)
    torch.cuda.synchronize()
    x_ref = x0.astype(np.float64).copy()
    pair.ora.decode_layer(0, kh, vh, x_ref, pos, cpos)
    err = max_rel(x_dev.cpu().numpy(), x_ref)
    log(f"  hidden max_rel={err:.3e}")
    assert err <= TOL
    _check_cache(kv, kh, vh, {(b, int(c)) for b, c in enumerate(cpos)})
